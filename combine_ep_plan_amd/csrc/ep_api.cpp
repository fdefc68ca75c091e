// C ABI of the dispatch/combine library: descriptor checks, plan workspace
// layout, device selection from the stream, and kernel launches.
//
// The device of every call is the stream's device, made current for the
// duration of the call and restored afterwards; the calling thread's current
// device is never assumed. In the same-node KV-transfer study "EFA の同じ
// ノード内の GPU 間通信: libfabric の shm と SAR" (sections 問題 and 直し方2),
// a transfer thread that never selected its GPU silently fell back to a slow
// path.
#include "ep.h"

#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <string>

#include "ep_kernels.hpp"
#include "ep_probe.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* msg) {
  g_last_error = msg;
  return code;
}

int fail_hip(hipError_t e, const char* where) {
  g_last_error = std::string(where) + ": " + hipGetErrorString(e);
  return EP_ERR_HIP;
}

constexpr int64_t kMaxWaves = (int64_t)1 << 26;  // grid.x * 64 threads < 2^32

int64_t bound_of(const ep_desc* d) {
  const int64_t L = d->n_experts / d->n_ranks;
  const int64_t m = d->topk > L ? d->topk : L;
  return (int64_t)d->n_ranks * d->tokens * m;
}

// Validate a descriptor and derive sizes. Returns EP_OK or a negative code.
int derive(const ep_desc* d, ep::Dims* o) {
  if (!d) return fail(EP_ERR_INVALID_ARG, "null descriptor");
  if (d->n_ranks <= 0 || d->tokens < 0 || d->hidden <= 0 || d->n_experts <= 0 || d->topk <= 0)
    return fail(EP_ERR_INVALID_ARG, "sizes must be positive (tokens may be 0)");
  if (d->n_experts % d->n_ranks != 0)
    return fail(EP_ERR_INVALID_ARG, "n_experts must be a multiple of n_ranks");
  if (d->payload != EP_PAYLOAD_BF16 && d->payload != EP_PAYLOAD_FP8_B128)
    return fail(EP_ERR_INVALID_ARG, "unknown payload");
  if (d->payload == EP_PAYLOAD_BF16 && d->hidden % 8 != 0)
    return fail(EP_ERR_INVALID_ARG, "bf16 payload needs hidden % 8 == 0");
  if (d->payload == EP_PAYLOAD_FP8_B128 && d->hidden % 128 != 0)
    return fail(EP_ERR_INVALID_ARG, "fp8 payload needs hidden % 128 == 0");
  if (d->cap_rows < 0) return fail(EP_ERR_INVALID_ARG, "cap_rows must be >= 0");
  if (d->n_experts > EP_MAX_EXPERTS) return fail(EP_ERR_UNSUPPORTED, "too many experts");
  if (d->topk > EP_MAX_TOPK) return fail(EP_ERR_UNSUPPORTED, "topk too large");
  const int64_t cap = d->cap_rows > 0 ? d->cap_rows : bound_of(d);
  const int64_t NTR = (int64_t)d->n_ranks * d->tokens * d->topk;
  // A zero capacity only arises from the bound with no tokens at all.
  if ((int64_t)d->n_ranks * cap >= ((int64_t)1 << 31))
    return fail(EP_ERR_UNSUPPORTED, "n_ranks * cap_rows must be < 2^31");
  if (NTR >= kMaxWaves) return fail(EP_ERR_UNSUPPORTED, "n_ranks * tokens * topk must be < 2^26");
  o->N = d->n_ranks;
  o->T = d->tokens;
  o->H = d->hidden;
  o->E = d->n_experts;
  o->R = d->topk;
  o->L = d->n_experts / d->n_ranks;
  o->payload = d->payload;
  o->planes = d->payload == EP_PAYLOAD_BF16 ? 1 : 2;
  o->cap = cap;
  o->TR = (int64_t)d->tokens * d->topk;
  o->NT = (int64_t)d->n_ranks * d->tokens;
  o->NTR = NTR;
  if (d->payload == EP_PAYLOAD_BF16) {
    o->row[0] = 2 * (int64_t)d->hidden;
    o->row[1] = 0;
  } else {
    o->row[0] = d->hidden;
    o->row[1] = 4 * (int64_t)(d->hidden / 128);
  }
  const int64_t nch = (o->TR + ep::kPlanChunk - 1) / ep::kPlanChunk;
  o->nchunks = (int)(nch > 0 ? nch : 1);
  // Windowed sender: windows of the largest power-of-two token count whose
  // rows fit kGatherSourceBytes.
  const int64_t tok_bytes = o->row[0] + o->row[1];
  const int64_t src_bytes = (int64_t)d->tokens * tok_bytes;
  o->win = 0;
  o->nwin = 0;
  if (src_bytes > ep::kGatherSourceBytes && src_bytes <= ep::kWindowSourceBytes &&
      NTR * tok_bytes <= ep::kWindowSendBytes) {
    int64_t w = 1;
    while (2 * w * tok_bytes <= ep::kGatherSourceBytes) w *= 2;
    o->win = (int)w;
    o->nwin = (int)((d->tokens + w - 1) / w);
  }
  // Bound on the copy grids: the row copies launch one wave per 1 KB piece
  // of a row (a plane under 1 KB counts as one piece), so one launch stays
  // under 2^26 waves: 2^32 work-items of 64 lanes, the most one dispatch
  // can hold.
  int64_t pieces = 0;
  for (int q = 0; q < o->planes; ++q) pieces += (o->row[q] + 1023) / 1024;
  if (NTR * pieces >= kMaxWaves)
    return fail(EP_ERR_UNSUPPORTED,
                "n_ranks * tokens * topk * (1 KB pieces per row) must be < 2^26");
  return EP_OK;
}

// Plan workspace: int32 arrays, each starting on a 256-byte boundary.
struct Layout {
  size_t off[14];
  size_t bytes;
};

Layout layout_of(const ep::Dims& d) {
  const size_t n[14] = {
      (size_t)d.N * d.E,                       // cnt
      (size_t)d.N * (d.E + 1),                 // send_off
      (size_t)d.NTR,                           // send_pos
      (size_t)d.N * (d.N + 1),                 // recv_off
      (size_t)d.N * (d.L + 1),                 // grp_off
      (size_t)d.NTR,                           // grp_pos
      (size_t)d.N * d.E,                       // src_off
      (size_t)d.NTR,                           // comb_row
      (size_t)d.NTR,                           // grp_slot
      (size_t)d.N * d.nchunks * d.E,           // chunk_cnt
      (size_t)d.NTR,                           // send_slot
      (size_t)2 * d.NTR,                       // recv_rows
      (size_t)d.NTR,                           // send_seg
      (size_t)2 * d.N * d.nwin * d.win * d.R,  // win_list (windowed sender only)
  };
  Layout l{};
  size_t at = 0;
  for (int i = 0; i < 14; ++i) {
    l.off[i] = at;
    at += (n[i] * sizeof(int32_t) + 255) & ~(size_t)255;
  }
  l.bytes = at > 0 ? at : 256;
  return l;
}

ep::PlanPtrs plan_ptrs(const ep::Dims& d, const void* ws) {
  const Layout l = layout_of(d);
  char* b = (char*)ws;
  ep::PlanPtrs p;
  p.cnt = (int32_t*)(b + l.off[0]);
  p.send_off = (int32_t*)(b + l.off[1]);
  p.send_pos = (int32_t*)(b + l.off[2]);
  p.recv_off = (int32_t*)(b + l.off[3]);
  p.grp_off = (int32_t*)(b + l.off[4]);
  p.grp_pos = (int32_t*)(b + l.off[5]);
  p.src_off = (int32_t*)(b + l.off[6]);
  p.comb_row = (int32_t*)(b + l.off[7]);
  p.grp_slot = (int32_t*)(b + l.off[8]);
  p.chunk_cnt = (int32_t*)(b + l.off[9]);
  p.send_slot = (int32_t*)(b + l.off[10]);
  p.recv_rows = (int32_t*)(b + l.off[11]);
  p.send_seg = (int32_t*)(b + l.off[12]);
  p.win_list = d.win > 0 ? (int32_t*)(b + l.off[13]) : nullptr;
  return p;
}

// Makes the stream's device current for the lifetime of the object.
class DeviceScope {
 public:
  explicit DeviceScope(hipStream_t s) {
    err_ = hipGetDevice(&prev_);
    if (err_ != hipSuccess) return;
    err_ = hipStreamGetDevice(s, &dev_);
    if (err_ != hipSuccess) return;
    if (dev_ != prev_) err_ = hipSetDevice(dev_);
  }
  ~DeviceScope() {
    if (err_ == hipSuccess && dev_ != prev_) (void)hipSetDevice(prev_);
  }
  hipError_t error() const { return err_; }
  int device() const { return dev_; }

 private:
  int prev_ = -1;
  int dev_ = -1;
  hipError_t err_ = hipSuccess;
};

// A non-empty buffer must be device (or managed) memory of the stream's GPU
// and, where the runtime reports the allocation's range, lie inside it for
// all `bytes`; an empty one (bytes == 0) is never touched and may be
// anything.
int check_ptr(const void* p, int dev, const char* name, int64_t bytes) {
  if (bytes == 0) return EP_OK;
  if (!p) return fail(EP_ERR_INVALID_ARG, (std::string("null pointer: ") + name).c_str());
  hipPointerAttribute_t a;
  std::memset(&a, 0, sizeof a);
  const hipError_t e = hipPointerGetAttributes(&a, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(EP_ERR_INVALID_ARG, (std::string("not device memory: ") + name).c_str());
  }
  if (a.type != hipMemoryTypeDevice && a.type != hipMemoryTypeManaged)
    return fail(EP_ERR_INVALID_ARG, (std::string("not device memory: ") + name).c_str());
  if (a.type == hipMemoryTypeDevice && a.device != dev)
    return fail(EP_ERR_DEVICE_MISMATCH,
                (std::string("buffer on another device: ") + name).c_str());
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)p) == hipSuccess && base != nullptr) {
    const uintptr_t end = (uintptr_t)base + size;
    if ((uintptr_t)p < (uintptr_t)base || (uint64_t)bytes > end - (uintptr_t)p)
      return fail(EP_ERR_INVALID_ARG,
                  (std::string("buffer smaller than the call needs: ") + name).c_str());
  } else {
    (void)hipGetLastError();
  }
  return EP_OK;
}

// rows: rows of every plane buffer (its bytes are rows * row bytes).
// Row buffers are moved with 16-byte vector accesses: their base must be
// 16-byte aligned (every row then is, row sizes being multiples of 16 or
// moved 4 bytes at a time).
int check_aligned16(const void* p, const char* name) {
  if (((uintptr_t)p & 15) != 0)
    return fail(EP_ERR_INVALID_ARG, (std::string("not 16-byte aligned: ") + name).c_str());
  return EP_OK;
}

int check_planes(const ep::Dims& d, const void* const* pl, int dev, const char* name,
                 int64_t rows) {
  if (!pl) return fail(EP_ERR_INVALID_ARG, (std::string("null plane array: ") + name).c_str());
  for (int q = 0; q < d.planes; ++q) {
    int rc = check_ptr(pl[q], dev, name, rows * d.row[q]);
    if (rc != EP_OK) return rc;
    rc = check_aligned16(pl[q], name);
    if (rc != EP_OK) return rc;
  }
  if (d.planes == 1 && pl[1] != nullptr)
    return fail(EP_ERR_INVALID_ARG, (std::string("plane 1 must be NULL for bf16: ") + name).c_str());
  return EP_OK;
}

// Common prologue: descriptor, device scope, workspace pointer.
#define EP_PROLOGUE(desc, stream, ws)                                    \
  ep::Dims dims;                                                         \
  {                                                                      \
    const int rc_ = derive(desc, &dims);                                 \
    if (rc_ != EP_OK) return rc_;                                        \
  }                                                                      \
  DeviceScope scope(stream);                                             \
  if (scope.error() != hipSuccess) return fail_hip(scope.error(), "device"); \
  {                                                                      \
    int rc_ = check_ptr(ws, scope.device(), "plan_ws", (int64_t)layout_of(dims).bytes); \
    if (rc_ == EP_OK) rc_ = check_aligned16(ws, "plan_ws");              \
    if (rc_ != EP_OK) return rc_;                                        \
  }                                                                      \
  const ep::PlanPtrs pp = plan_ptrs(dims, ws);

#define EP_CHECK(expr)            \
  do {                            \
    const int rc_ = (expr);       \
    if (rc_ != EP_OK) return rc_; \
  } while (0)

}  // namespace

extern "C" {

int64_t ep_recv_bound(const ep_desc* d) {
  ep::Dims dims;
  if (derive(d, &dims) != EP_OK) return -1;
  return bound_of(d);
}

int64_t ep_capacity(const ep_desc* d) {
  ep::Dims dims;
  if (derive(d, &dims) != EP_OK) return -1;
  return dims.cap;
}

int ep_num_planes(const ep_desc* d) {
  ep::Dims dims;
  if (derive(d, &dims) != EP_OK) return -1;
  return dims.planes;
}

int64_t ep_row_bytes(const ep_desc* d, int plane) {
  ep::Dims dims;
  if (derive(d, &dims) != EP_OK) return -1;
  if (plane < 0 || plane > 1) return 0;
  return dims.row[plane];
}

size_t ep_plan_bytes(const ep_desc* d) {
  ep::Dims dims;
  if (derive(d, &dims) != EP_OK) return 0;
  return layout_of(dims).bytes;
}

int ep_plan_views(const ep_desc* d, void* plan_ws, ep_plan_view* v) {
  ep::Dims dims;
  EP_CHECK(derive(d, &dims));
  if (!plan_ws || !v) return fail(EP_ERR_INVALID_ARG, "null workspace or view");
  const ep::PlanPtrs p = plan_ptrs(dims, plan_ws);
  v->cnt = p.cnt;
  v->send_off = p.send_off;
  v->send_pos = p.send_pos;
  v->recv_off = p.recv_off;
  v->grp_off = p.grp_off;
  v->grp_pos = p.grp_pos;
  v->src_off = p.src_off;
  v->comb_row = p.comb_row;
  v->grp_slot = p.grp_slot;
  v->send_slot = p.send_slot;
  v->recv_rows = p.recv_rows;
  v->send_seg = p.send_seg;
  v->win_list = p.win_list;
  return EP_OK;
}

int ep_plan(const ep_desc* d, const int32_t* topk_idx, void* plan_ws, int32_t* status,
            hipStream_t stream) {
  EP_PROLOGUE(d, stream, plan_ws);
  EP_CHECK(check_ptr(status, scope.device(), "status", 4));
  EP_CHECK(check_ptr(topk_idx, scope.device(), "topk_idx", 4 * dims.NTR));
  const hipError_t e = ep::launch_plan(dims, topk_idx, pp, status, stream);
  if (e != hipSuccess) return fail_hip(e, "ep_plan");
  return EP_OK;
}

int ep_dispatch(const ep_desc* d, const int32_t* topk_idx, const void* const x[2],
                void* plan_ws, void* const send[2], void* const grouped[2], int32_t* status,
                hipStream_t stream) {
  EP_PROLOGUE(d, stream, plan_ws);
  EP_CHECK(check_ptr(status, scope.device(), "status", 4));
  EP_CHECK(check_ptr(topk_idx, scope.device(), "topk_idx", 4 * dims.NTR));
  EP_CHECK(check_planes(dims, (const void* const*)x, scope.device(), "x", dims.NT));
  EP_CHECK(check_planes(dims, (const void* const*)send, scope.device(), "send", dims.NTR));
  EP_CHECK(check_planes(dims, (const void* const*)grouped, scope.device(), "grouped", dims.N * dims.cap));
  const hipError_t e = ep::launch_dispatch(dims, topk_idx, x, pp, send, grouped, status, stream);
  if (e != hipSuccess) return fail_hip(e, "ep_dispatch");
  return EP_OK;
}

int ep_dispatch_pack(const ep_desc* d, const void* const x[2], const void* plan_ws,
                     void* const send[2], hipStream_t stream) {
  EP_PROLOGUE(d, stream, plan_ws);
  EP_CHECK(check_planes(dims, (const void* const*)x, scope.device(), "x", dims.NT));
  EP_CHECK(check_planes(dims, (const void* const*)send, scope.device(), "send", dims.NTR));
  const hipError_t e = ep::launch_pack(dims, x, pp, send, stream);
  if (e != hipSuccess) return fail_hip(e, "ep_dispatch_pack");
  return EP_OK;
}

int ep_dispatch_pack_quant(const ep_desc* d, const uint16_t* x, const void* plan_ws,
                           void* const send[2], hipStream_t stream) {
  EP_PROLOGUE(d, stream, plan_ws);
  if (dims.payload != EP_PAYLOAD_FP8_B128)
    return fail(EP_ERR_INVALID_ARG, "ep_dispatch_pack_quant needs the fp8 payload descriptor");
  // one wave per 1024-value segment of a token row
  if (dims.NT * (((int64_t)dims.H + 1023) / 1024) >= kMaxWaves)
    return fail(EP_ERR_UNSUPPORTED, "tokens x 1024-value row segments must be < 2^26");
  EP_CHECK(check_ptr(x, scope.device(), "x", dims.NT * 2 * (int64_t)dims.H));
  EP_CHECK(check_aligned16(x, "x"));
  EP_CHECK(check_planes(dims, (const void* const*)send, scope.device(), "send", dims.NTR));
  const hipError_t e = ep::launch_pack_quant(dims, x, pp, send, stream);
  if (e != hipSuccess) return fail_hip(e, "ep_dispatch_pack_quant");
  return EP_OK;
}

int ep_dispatch_quant(const ep_desc* d, const int32_t* topk_idx, const uint16_t* x,
                      void* plan_ws, void* const send[2], void* const grouped[2], int32_t* status,
                      hipStream_t stream) {
  EP_PROLOGUE(d, stream, plan_ws);
  if (dims.payload != EP_PAYLOAD_FP8_B128)
    return fail(EP_ERR_INVALID_ARG, "ep_dispatch_quant needs the fp8 payload descriptor");
  if (dims.NT * (((int64_t)dims.H + 1023) / 1024) >= kMaxWaves)
    return fail(EP_ERR_UNSUPPORTED, "tokens x 1024-value row segments must be < 2^26");
  EP_CHECK(check_ptr(status, scope.device(), "status", 4));
  EP_CHECK(check_ptr(topk_idx, scope.device(), "topk_idx", 4 * dims.NTR));
  EP_CHECK(check_ptr(x, scope.device(), "x", dims.NT * 2 * (int64_t)dims.H));
  EP_CHECK(check_aligned16(x, "x"));
  EP_CHECK(check_planes(dims, (const void* const*)send, scope.device(), "send", dims.NTR));
  EP_CHECK(check_planes(dims, (const void* const*)grouped, scope.device(), "grouped", dims.N * dims.cap));
  const hipError_t e = ep::launch_dispatch_quant(dims, topk_idx, x, pp, send, grouped, status, stream);
  if (e != hipSuccess) return fail_hip(e, "ep_dispatch_quant");
  return EP_OK;
}

int ep_dispatch_transfer(const ep_desc* d, const void* const send[2], const void* plan_ws,
                         void* const recv[2], hipStream_t stream) {
  EP_PROLOGUE(d, stream, plan_ws);
  EP_CHECK(check_planes(dims, (const void* const*)send, scope.device(), "send", dims.NTR));
  EP_CHECK(check_planes(dims, (const void* const*)recv, scope.device(), "recv", dims.N * dims.cap));
  const hipError_t e = ep::launch_transfer(dims, send, pp, recv, stream);
  if (e != hipSuccess) return fail_hip(e, "ep_dispatch_transfer");
  return EP_OK;
}

int ep_dispatch_unpack(const ep_desc* d, const void* const recv[2], const void* plan_ws,
                       void* const grouped[2], hipStream_t stream) {
  EP_PROLOGUE(d, stream, plan_ws);
  EP_CHECK(check_planes(dims, (const void* const*)recv, scope.device(), "recv", dims.N * dims.cap));
  EP_CHECK(check_planes(dims, (const void* const*)grouped, scope.device(), "grouped", dims.N * dims.cap));
  const hipError_t e = ep::launch_unpack(dims, recv, pp, grouped, stream);
  if (e != hipSuccess) return fail_hip(e, "ep_dispatch_unpack");
  return EP_OK;
}

int ep_dispatch_recv(const ep_desc* d, const void* const send[2], const void* plan_ws,
                     void* const grouped[2], hipStream_t stream) {
  EP_PROLOGUE(d, stream, plan_ws);
  EP_CHECK(check_planes(dims, (const void* const*)send, scope.device(), "send", dims.NTR));
  EP_CHECK(check_planes(dims, (const void* const*)grouped, scope.device(), "grouped", dims.N * dims.cap));
  const hipError_t e = ep::launch_recv(dims, send, pp, grouped, stream);
  if (e != hipSuccess) return fail_hip(e, "ep_dispatch_recv");
  return EP_OK;
}

// Private regions: P rows per (destination, source) pair, P in [0, T R].
int check_priv(const ep::Dims& d, void* const priv[2], int32_t P, int dev) {
  if (P < 0 || P > d.TR) return fail(EP_ERR_INVALID_ARG, "priv_rows must be in [0, tokens * topk]");
  if (P == 0) return EP_OK;
  return check_planes(d, (const void* const*)priv, dev, "priv", (int64_t)d.N * d.N * P);
}

int ep_dispatch_send_plan(const ep_desc* d, const int32_t* topk_idx, void* plan_ws,
                          int32_t* status, hipStream_t stream) {
  EP_PROLOGUE(d, stream, plan_ws);
  EP_CHECK(check_ptr(status, scope.device(), "status", 4));
  EP_CHECK(check_ptr(topk_idx, scope.device(), "topk_idx", 4 * dims.NTR));
  const hipError_t e = ep::launch_plan_local(dims, topk_idx, pp, status, stream);
  if (e != hipSuccess) return fail_hip(e, "ep_dispatch_send_plan");
  return EP_OK;
}

int ep_dispatch_send_pack(const ep_desc* d, const int32_t* topk_idx, const void* const x[2],
                          const void* plan_ws, void* const send[2], void* const priv[2],
                          int32_t priv_rows, hipStream_t stream) {
  EP_PROLOGUE(d, stream, plan_ws);
  EP_CHECK(check_ptr(topk_idx, scope.device(), "topk_idx", 4 * dims.NTR));
  EP_CHECK(check_planes(dims, (const void* const*)x, scope.device(), "x", dims.NT));
  EP_CHECK(check_planes(dims, (const void* const*)send, scope.device(), "send", dims.NTR));
  EP_CHECK(check_priv(dims, priv, priv_rows, scope.device()));
  const hipError_t e = ep::launch_pack_split(dims, topk_idx, x, pp, send, priv, priv_rows, stream);
  if (e != hipSuccess) return fail_hip(e, "ep_dispatch_send_pack");
  return EP_OK;
}

int ep_dispatch_recv_plan(const ep_desc* d, void* plan_ws, int32_t* status, hipStream_t stream) {
  EP_PROLOGUE(d, stream, plan_ws);
  EP_CHECK(check_ptr(status, scope.device(), "status", 4));
  const hipError_t e = ep::launch_plan_exchange(dims, pp, status, stream);
  if (e != hipSuccess) return fail_hip(e, "ep_dispatch_recv_plan");
  return EP_OK;
}

int ep_dispatch_recv_pull(const ep_desc* d, const void* const send[2], void* const priv[2],
                          int32_t priv_rows, const void* plan_ws, void* const grouped[2],
                          hipStream_t stream) {
  EP_PROLOGUE(d, stream, plan_ws);
  EP_CHECK(check_planes(dims, (const void* const*)send, scope.device(), "send", dims.NTR));
  EP_CHECK(check_priv(dims, priv, priv_rows, scope.device()));
  EP_CHECK(check_planes(dims, (const void* const*)grouped, scope.device(), "grouped", dims.N * dims.cap));
  const hipError_t e = ep::launch_recv_split(dims, send, priv, priv_rows, pp, grouped, stream);
  if (e != hipSuccess) return fail_hip(e, "ep_dispatch_recv_pull");
  return EP_OK;
}

int ep_dispatch_send(const ep_desc* d, const int32_t* topk_idx, const void* const x[2],
                     void* plan_ws, void* const send[2], void* const priv[2], int32_t priv_rows,
                     int32_t* status, hipStream_t stream) {
  // Check everything before enqueueing the first half.
  {
    EP_PROLOGUE(d, stream, plan_ws);
    EP_CHECK(check_ptr(status, scope.device(), "status", 4));
    EP_CHECK(check_ptr(topk_idx, scope.device(), "topk_idx", 4 * dims.NTR));
    EP_CHECK(check_planes(dims, (const void* const*)x, scope.device(), "x", dims.NT));
    EP_CHECK(check_planes(dims, (const void* const*)send, scope.device(), "send", dims.NTR));
    EP_CHECK(check_priv(dims, priv, priv_rows, scope.device()));
    (void)pp;
  }
  EP_CHECK(ep_dispatch_send_plan(d, topk_idx, plan_ws, status, stream));
  return ep_dispatch_send_pack(d, topk_idx, x, plan_ws, send, priv, priv_rows, stream);
}

int ep_dispatch_recv_split(const ep_desc* d, const void* const send[2], void* const priv[2],
                           int32_t priv_rows, void* plan_ws, void* const grouped[2],
                           int32_t* status, hipStream_t stream) {
  // Check everything before enqueueing the first half.
  {
    EP_PROLOGUE(d, stream, plan_ws);
    EP_CHECK(check_ptr(status, scope.device(), "status", 4));
    EP_CHECK(check_planes(dims, (const void* const*)send, scope.device(), "send", dims.NTR));
    EP_CHECK(check_priv(dims, priv, priv_rows, scope.device()));
    EP_CHECK(check_planes(dims, (const void* const*)grouped, scope.device(), "grouped",
                          dims.N * dims.cap));
    (void)pp;
  }
  EP_CHECK(ep_dispatch_recv_plan(d, plan_ws, status, stream));
  return ep_dispatch_recv_pull(d, send, priv, priv_rows, plan_ws, grouped, stream);
}

int ep_expert_stub(const ep_desc* d, const void* const grouped[2], const float* alpha,
                   const void* plan_ws, uint16_t* expert_out, hipStream_t stream) {
  EP_PROLOGUE(d, stream, plan_ws);
  EP_CHECK(check_planes(dims, (const void* const*)grouped, scope.device(), "grouped", dims.N * dims.cap));
  EP_CHECK(check_ptr(expert_out, scope.device(), "expert_out", dims.N * dims.cap * 2 * dims.H));
  EP_CHECK(check_aligned16(expert_out, "expert_out"));
  if (alpha) {
    if (dims.payload != EP_PAYLOAD_BF16)
      return fail(EP_ERR_INVALID_ARG, "alpha applies to the bf16 payload only");
    EP_CHECK(check_ptr(alpha, scope.device(), "alpha", 4 * (int64_t)dims.E));
  }
  const hipError_t e = ep::launch_expert_stub(dims, grouped, alpha, pp, expert_out, stream);
  if (e != hipSuccess) return fail_hip(e, "ep_expert_stub");
  return EP_OK;
}

int ep_combine(const ep_desc* d, const uint16_t* expert_out, const float* weights,
               const void* plan_ws, uint16_t* out, hipStream_t stream) {
  EP_PROLOGUE(d, stream, plan_ws);
  EP_CHECK(check_ptr(expert_out, scope.device(), "expert_out", dims.N * dims.cap * 2 * dims.H));
  EP_CHECK(check_ptr(out, scope.device(), "out", dims.NT * 2 * dims.H));
  EP_CHECK(check_ptr(weights, scope.device(), "weights", 4 * dims.NTR));
  EP_CHECK(check_aligned16(expert_out, "expert_out"));
  EP_CHECK(check_aligned16(out, "out"));
  const hipError_t e = ep::launch_combine(dims, expert_out, weights, pp, out, stream);
  if (e != hipSuccess) return fail_hip(e, "ep_combine");
  return EP_OK;
}

int ep_combine_presum(const ep_desc* d, const uint16_t* expert_out, const float* weights,
                      const void* plan_ws, uint16_t* partial, uint16_t* out, hipStream_t stream) {
  EP_PROLOGUE(d, stream, plan_ws);
  EP_CHECK(check_ptr(expert_out, scope.device(), "expert_out", dims.N * dims.cap * 2 * dims.H));
  EP_CHECK(check_ptr(partial, scope.device(), "partial", dims.NTR * 2 * dims.H));
  EP_CHECK(check_ptr(out, scope.device(), "out", dims.NT * 2 * dims.H));
  EP_CHECK(check_ptr(weights, scope.device(), "weights", 4 * dims.NTR));
  EP_CHECK(check_aligned16(expert_out, "expert_out"));
  EP_CHECK(check_aligned16(partial, "partial"));
  EP_CHECK(check_aligned16(out, "out"));
  const hipError_t e = ep::launch_combine_presum(dims, expert_out, weights, pp, partial, out, stream);
  if (e != hipSuccess) return fail_hip(e, "ep_combine_presum");
  return EP_OK;
}

// ---------------------------------------------------------------------------
// KV-block push
// ---------------------------------------------------------------------------

int64_t ep_kv_plan(int64_t n, int64_t tok, int64_t bs_src, const int32_t* src_blocks,
                   int64_t bs_dst, const int32_t* dst_blocks, int32_t merge,
                   ep_kv_region* regions, int64_t max_regions) {
  if (n < 0 || tok <= 0 || tok % 16 != 0 || bs_src <= 0 || bs_dst <= 0)
    return fail(EP_ERR_INVALID_ARG, "ep_kv_plan: bad sizes (token_bytes must be a positive multiple of 16)");
  if (n > 0 && (!src_blocks || !dst_blocks || !regions))
    return fail(EP_ERR_INVALID_ARG, "ep_kv_plan: null table or output");
  int64_t m = 0;
  // Walk the request in spans that stay inside one source block and one
  // destination block (contiguous on both sides by construction); a span
  // extends the previous region when both its addresses continue it.
  for (int64_t i = 0; i < n;) {
    const int64_t sb = i / bs_src, so = i % bs_src, db = i / bs_dst, dof = i % bs_dst;
    const int32_t bsrc = src_blocks[sb], bdst = dst_blocks[db];
    if (bsrc < 0 || bdst < 0) return fail(EP_ERR_INVALID_ARG, "ep_kv_plan: negative block id");
    int64_t span = bs_src - so;
    if (bs_dst - dof < span) span = bs_dst - dof;
    if (n - i < span) span = n - i;
    const int64_t src_off = ((int64_t)bsrc * bs_src + so) * tok;
    const int64_t dst_off = ((int64_t)bdst * bs_dst + dof) * tok;
    ep_kv_region* prev = m > 0 ? &regions[m - 1] : nullptr;
    if (merge && prev && prev->src_off + prev->bytes == src_off &&
        prev->dst_off + prev->bytes == dst_off) {
      prev->bytes += span * tok;
    } else {
      if (m >= max_regions) return fail(EP_ERR_INVALID_ARG, "ep_kv_plan: max_regions too small");
      regions[m] = ep_kv_region{src_off, dst_off, span * tok, i * tok};
      ++m;
    }
    i += span;
  }
  return m;
}

namespace {

int kv_checks(int32_t ranks, const ep_kv_region* regions, int64_t m, int64_t total,
              const void* src, int64_t src_rank_bytes, void* dst, int64_t dst_rank_bytes,
              int32_t* notify, int32_t* status, int dev) {
  if (ranks < 1 || m < 0 || total < 0 || total % 16 != 0 || src_rank_bytes < 0 ||
      dst_rank_bytes < 0 || src_rank_bytes % 16 != 0 || dst_rank_bytes % 16 != 0)
    return fail(EP_ERR_INVALID_ARG, "ep_kv_push: bad sizes (bytes must be multiples of 16)");
  if (((uintptr_t)src | (uintptr_t)dst) & 15)
    return fail(EP_ERR_INVALID_ARG, "ep_kv_push: pools must be 16-byte aligned");
  const int64_t pieces = (total + ep::kv_piece_bytes() - 1) / ep::kv_piece_bytes();
  if (pieces >= kMaxWaves / ranks) return fail(EP_ERR_UNSUPPORTED, "ep_kv_push: request too large");
  EP_CHECK(check_ptr(regions, dev, "regions", m * (int64_t)sizeof(ep_kv_region)));
  EP_CHECK(check_ptr(src, dev, "src_pool", src_rank_bytes * ranks));
  EP_CHECK(check_ptr(dst, dev, "dst_pool", dst_rank_bytes * ranks));
  EP_CHECK(check_ptr(notify, dev, "notify", 4));
  EP_CHECK(check_ptr(status, dev, "status", 4));
  return EP_OK;
}

// Device memory of `dev` (at least `bytes` of it), or pinned host memory.
int check_bounce(const void* p, int dev, int64_t bytes) {
  if (!p) return fail(EP_ERR_INVALID_ARG, "null pointer: bounce");
  if (((uintptr_t)p) & 15) return fail(EP_ERR_INVALID_ARG, "bounce must be 16-byte aligned");
  hipPointerAttribute_t a;
  std::memset(&a, 0, sizeof a);
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();
    return fail(EP_ERR_INVALID_ARG, "bounce is neither device nor pinned host memory");
  }
  if (a.type == hipMemoryTypeHost) return EP_OK;
  return check_ptr(p, dev, "bounce", bytes);
}

}  // namespace

int ep_kv_push(int32_t ranks, const ep_kv_region* regions, int64_t m, int64_t total,
               const void* src, int64_t src_rank_bytes, void* dst, int64_t dst_rank_bytes,
               int32_t* notify, int32_t* status, hipStream_t stream) {
  DeviceScope scope(stream);
  if (scope.error() != hipSuccess) return fail_hip(scope.error(), "device");
  EP_CHECK(kv_checks(ranks, regions, m, total, src, src_rank_bytes, dst, dst_rank_bytes, notify,
                     status, scope.device()));
  const hipError_t e = ep::launch_kv_push(ranks, regions, m, total, src, src_rank_bytes, dst,
                                          dst_rank_bytes, notify, status, stream);
  if (e != hipSuccess) return fail_hip(e, "ep_kv_push");
  return EP_OK;
}

int ep_kv_push_staged(int32_t ranks, const ep_kv_region* regions, int64_t m, int64_t total,
                      const void* src, int64_t src_rank_bytes, void* dst, int64_t dst_rank_bytes,
                      void* bounce, int32_t slots, int32_t* notify, int32_t* status,
                      hipStream_t stream) {
  DeviceScope scope(stream);
  if (scope.error() != hipSuccess) return fail_hip(scope.error(), "device");
  EP_CHECK(kv_checks(ranks, regions, m, total, src, src_rank_bytes, dst, dst_rank_bytes, notify,
                     status, scope.device()));
  if (slots < 1 || slots > ep::kKvStaticSlots)
    return fail(EP_ERR_INVALID_ARG, "bounce_slots must be in [1, 64]");
  EP_CHECK(check_bounce(bounce, scope.device(), (int64_t)slots * ep::kKvSlotBytes));
  const hipError_t e = ep::launch_kv_push_staged(ranks, regions, m, total, src, src_rank_bytes,
                                                 dst, dst_rank_bytes, bounce,
                                                 (int64_t)slots * ep::kKvSlotBytes, notify, status,
                                                 stream);
  if (e != hipSuccess) return fail_hip(e, "ep_kv_push_staged");
  return EP_OK;
}

int ep_kv_push_staged_static(int32_t ranks, const ep_kv_region* regions, int64_t m,
                             int64_t total, const void* src, int64_t src_rank_bytes, void* dst,
                             int64_t dst_rank_bytes, int32_t slots, int32_t* notify,
                             int32_t* status, hipStream_t stream) {
  DeviceScope scope(stream);
  if (scope.error() != hipSuccess) return fail_hip(scope.error(), "device");
  EP_CHECK(kv_checks(ranks, regions, m, total, src, src_rank_bytes, dst, dst_rank_bytes, notify,
                     status, scope.device()));
  if (slots < 1 || slots > ep::kKvStaticSlots)
    return fail(EP_ERR_INVALID_ARG,
                "bounce_slots must be in [1, 64]: the library's static bounce area holds 64 "
                "slots of 32 KiB");
  // The stream's device is current here (DeviceScope), as the lookup needs.
  void* bounce = nullptr;
  hipError_t e = ep::kv_static_bounce(scope.device(), &bounce);
  if (e != hipSuccess) return fail_hip(e, "ep_kv_push_staged_static: static bounce address");
  e = ep::launch_kv_push_staged(ranks, regions, m, total, src, src_rank_bytes, dst,
                                dst_rank_bytes, bounce, (int64_t)slots * ep::kKvSlotBytes, notify,
                                status, stream);
  if (e != hipSuccess) return fail_hip(e, "ep_kv_push_staged_static");
  return EP_OK;
}

int ep_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  if (bytes % 16 != 0) return fail(EP_ERR_INVALID_ARG, "bytes must be a multiple of 16");
  if (bytes / 16 >= (size_t)kMaxWaves * 64 * 7)
    return fail(EP_ERR_UNSUPPORTED, "copy too large");
  DeviceScope scope(stream);
  if (scope.error() != hipSuccess) return fail_hip(scope.error(), "device");
  EP_CHECK(check_ptr(dst, scope.device(), "dst", (int64_t)bytes));
  EP_CHECK(check_ptr(src, scope.device(), "src", (int64_t)bytes));
  const hipError_t e = ep::launch_probe_copy(dst, src, bytes, stream);
  if (e != hipSuccess) return fail_hip(e, "ep_probe_copy");
  return EP_OK;
}

int ep_probe_pattern(void* dst, const void* src, const int32_t* table, int64_t rows,
                     int64_t indexed_rows, int64_t row_bytes, int64_t piece_bytes, int fan_in,
                     int in_flight, int mode, int flags, int64_t waves, hipStream_t stream) {
  const bool scatter = mode == EP_PROBE_SCATTER || mode == EP_PROBE_SCATTER_WIDE;
  if (mode != EP_PROBE_COPY && mode != EP_PROBE_FILL && mode != EP_PROBE_READ && !scatter)
    return fail(EP_ERR_INVALID_ARG, "unknown probe mode");
  if (flags & ~(EP_PROBE_NT_LOADS | EP_PROBE_XCD | EP_PROBE_ONE_WAVE))
    return fail(EP_ERR_INVALID_ARG, "unknown probe flags");
  if (rows < 0 || indexed_rows < 0 || waves < 0)
    return fail(EP_ERR_INVALID_ARG, "rows, indexed_rows and waves must be >= 0");
  if (piece_bytes <= 0 || piece_bytes % 1024 != 0 || row_bytes <= 0 ||
      row_bytes % piece_bytes != 0)
    return fail(EP_ERR_INVALID_ARG,
                "piece_bytes must be a positive multiple of 1024 that divides row_bytes");
  const bool fans = mode == EP_PROBE_COPY || scatter;
  if (fans ? (fan_in != 1 && fan_in != 2 && fan_in != 4 && fan_in != 8) : fan_in != 1)
    return fail(EP_ERR_INVALID_ARG, "fan_in must be 1, 2, 4 or 8 (copy, scatter) or 1");
  if ((in_flight != 1 && in_flight != 2 && in_flight != 4 && in_flight != 8) ||
      fan_in % in_flight != 0 || (scatter && in_flight != 1))
    return fail(EP_ERR_INVALID_ARG,
                "in_flight must be 1, 2, 4 or 8 and divide fan_in (1 for a scatter)");
  if (waves > 0 && (flags & EP_PROBE_XCD))
    return fail(EP_ERR_INVALID_ARG, "the XCD renumbering applies to one piece per wave only");
  if (ep::probe_inflight((int)piece_bytes, mode == EP_PROBE_SCATTER_WIDE ? 2 : in_flight) == 0)
    return fail(EP_ERR_UNSUPPORTED, "no probe kernel for this piece size and in_flight");
  if (row_bytes > ((int64_t)1 << 29) || rows * (row_bytes / piece_bytes) >= ((int64_t)1 << 31) ||
      indexed_rows >= ((int64_t)1 << 31) || waves >= kMaxWaves)
    return fail(EP_ERR_UNSUPPORTED, "probe too large");
  const bool reads = mode != EP_PROBE_FILL;
  const bool indexed = mode != EP_PROBE_FILL;  // the table indexes src, or dst for a scatter
  if (indexed && rows > 0) {
    if (table == nullptr && indexed_rows < rows * fan_in)
      return fail(EP_ERR_INVALID_ARG, "indexed_rows must cover rows * fan_in without a table");
    if (table != nullptr && indexed_rows < 1)
      return fail(EP_ERR_INVALID_ARG, "indexed_rows must be >= 1");
  }
  int64_t dst_bytes = rows * row_bytes, src_bytes = indexed_rows * row_bytes;
  if (mode == EP_PROBE_READ) dst_bytes = rows > 0 ? 256 : 0;
  if (scatter) {
    dst_bytes = rows > 0 ? indexed_rows * row_bytes : 0;
    src_bytes = rows * row_bytes * (mode == EP_PROBE_SCATTER_WIDE ? 2 : 1);
  }
  DeviceScope scope(stream);
  if (scope.error() != hipSuccess) return fail_hip(scope.error(), "device");
  EP_CHECK(check_ptr(dst, scope.device(), "dst", dst_bytes));
  if (reads && rows > 0) {
    EP_CHECK(check_ptr(src, scope.device(), "src", src_bytes));
    if (table != nullptr)
      EP_CHECK(check_ptr(table, scope.device(), "table", rows * fan_in * 4));
  }
  ep::ProbeShape sh{};
  sh.dst = dst;
  sh.src = reads ? src : nullptr;
  sh.table = reads ? table : nullptr;
  sh.rows = (int32_t)rows;
  sh.indexed_rows = (int32_t)indexed_rows;
  sh.row_bytes = (int32_t)row_bytes;
  sh.piece_bytes = (int32_t)piece_bytes;
  sh.fan_in = fan_in;
  sh.in_flight = in_flight;
  sh.mode = mode;
  sh.nt_loads = (flags & EP_PROBE_NT_LOADS) != 0;
  sh.xcd = (flags & EP_PROBE_XCD) != 0;
  sh.one_wave = (flags & EP_PROBE_ONE_WAVE) != 0;
  sh.waves = (int32_t)waves;
  const hipError_t e = ep::launch_probe_pattern(sh, stream);
  if (e != hipSuccess) return fail_hip(e, "ep_probe_pattern");
  return EP_OK;
}

const char* ep_status_string(int code) {
  switch (code) {
    case EP_OK: return "ok";
    case EP_ERR_INVALID_ARG: return "invalid argument";
    case EP_ERR_UNSUPPORTED: return "unsupported size";
    case EP_ERR_DEVICE_MISMATCH: return "buffer on another device";
    case EP_ERR_HIP: return "HIP runtime error";
    case EP_STATUS_BAD_EXPERT: return "expert id out of range (slot dropped)";
    case EP_STATUS_CAPACITY: return "receive capacity exceeded (rows dropped)";
    case EP_STATUS_BAD_EXPERT | EP_STATUS_CAPACITY:
      return "expert id out of range and receive capacity exceeded";
    case EP_STATUS_BAD_REGION: return "KV region outside its pools (skipped)";
    default: return "unknown code";
  }
}

const char* ep_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
