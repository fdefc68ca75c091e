// Host-side launcher of the access-pattern probe (ep_probe.hip). Sizes are
// validated by the C ABI layer before it is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ep {

enum ProbeMode {
  kProbeCopy = 0,
  kProbeFill = 1,
  kProbeRead = 2,
  kProbeScatter = 3,
  kProbeScatterWide = 4
};

struct ProbeShape {
  void* dst;
  const void* src;
  const int32_t* table;  // row per (walked row, input or output), or null
  int32_t rows;          // rows walked: output rows (copy, fill), rows read (read, scatter)
  int32_t indexed_rows;  // rows of the buffer the table indexes (src; dst for scatter)
  int32_t row_bytes;     // multiple of piece_bytes
  int32_t piece_bytes;   // multiple of 1024: the bytes one wave moves
  int32_t fan_in;        // source rows per output row (copy), output rows per source row
                         // (scatter): 1, 2, 4 or 8
  int32_t in_flight;     // of them loaded together (divides fan_in)
  int32_t mode;          // ProbeMode
  bool nt_loads;         // non-temporal loads (else ordinary cached ones)
  bool xcd;              // renumber blocks per XCD
  bool one_wave;         // workgroups of one wave (else four)
  int32_t waves;         // 0: one piece per wave; > 0: that many waves, grid-stride
};

// Chunks per lane kept in flight for a shape (0 if no kernel fits it).
int probe_inflight(int piece_bytes, int in_flight);

hipError_t launch_probe_pattern(const ProbeShape& s, hipStream_t stream);

}  // namespace ep
