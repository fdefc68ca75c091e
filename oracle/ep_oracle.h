/*
 * CPU oracle for MoE expert-parallel dispatch/combine: TEST INFRASTRUCTURE.
 * Used only by the tests, the smoke check and the benchmark's CPU-baseline
 * leg. It shares no code, header or table with the HIP library.
 *
 * Notation: N ranks, T tokens per rank, E experts, R choices per token,
 * L = E/N experts per rank, cap = rows per destination buffer.
 * Arrays are dense row-major in the shapes given beside each function in
 * ep_oracle.c.
 */
#ifndef EP_ORACLE_H
#define EP_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_STATUS_BAD_EXPERT 1
#define ORACLE_STATUS_CAPACITY 2

float oracle_bf16_to_f32(uint16_t b);
uint16_t oracle_f64_to_bf16(double v);
uint16_t oracle_f32_to_bf16(float f);
float oracle_e4m3_to_f32(uint8_t c);
uint8_t oracle_f32_to_e4m3(float v);
void oracle_quantize_b128(int H, const uint16_t *x, uint8_t *codes, float *scales);
void oracle_dispatch_pack_quant(int N, int T, int R, int H, const uint16_t *x,
                                const int32_t *send_pos, uint8_t *codes,
                                float *scales);

int64_t oracle_recv_bound(int N, int T, int E, int R);

int oracle_plan(int N, int T, int E, int R, int64_t cap,
                const int32_t *idx, int32_t *cnt, int32_t *send_off,
                int32_t *send_pos, int32_t *recv_off, int32_t *grp_off,
                int32_t *grp_pos, int32_t *status);

void oracle_dispatch_pack(int N, int T, int R, int64_t row,
                          const uint8_t *x, const int32_t *send_pos,
                          uint8_t *send);
void oracle_transfer(int N, int T, int E, int R, int64_t row,
                     int64_t recv_rows, const uint8_t *send,
                     const int32_t *send_off, const int32_t *recv_off,
                     uint8_t *recv);
void oracle_unpack(int N, int T, int E, int R, int64_t row,
                   int64_t recv_rows, int64_t cap, const uint8_t *recv,
                   const int32_t *cnt, const int32_t *send_off,
                   const int32_t *recv_off, const int32_t *grp_off,
                   uint8_t *grouped);

void oracle_expert_bf16(int H, const uint16_t *in, const float *alpha, int e,
                        uint16_t *out);
void oracle_expert_fp8(int H, const uint8_t *codes, const float *scales,
                       uint16_t *out);
void oracle_expert_op(int N, int E, int H, int64_t cap, int payload,
                      const void *grouped0, const void *grouped1,
                      const float *alpha, const int32_t *grp_off,
                      uint16_t *y);

void oracle_combine_token(int H, int R, const float *w,
                          const uint16_t *const *rows, uint16_t *out);
void oracle_combine(int N, int T, int E, int R, int H, int64_t cap,
                    const int32_t *idx, const int32_t *grp_pos,
                    const uint16_t *y, const float *w, uint16_t *out);

void oracle_combine_presum_token(int H, int R, const float *w,
                                 const uint16_t *const *rows, const int *rank,
                                 uint16_t *partial, uint16_t *out);
void oracle_combine_presum(int N, int T, int E, int R, int H, int64_t cap,
                           const int32_t *idx, const int32_t *grp_pos,
                           const uint16_t *y, const float *w, uint16_t *partial,
                           uint16_t *out);

int64_t oracle_kv_regions(int64_t n, int64_t tok, int64_t bs_src,
                          const int32_t *src_blocks, int64_t bs_dst,
                          const int32_t *dst_blocks, int64_t *src_off,
                          int64_t *dst_off, int64_t *bytes);
void oracle_kv_copy(int ranks, int64_t m, const int64_t *src_off,
                    const int64_t *dst_off, const int64_t *bytes,
                    const uint8_t *src, int64_t src_rank_bytes, uint8_t *dst,
                    int64_t dst_rank_bytes);

int oracle_rounding_mode_is_nearest(void);

#ifdef __cplusplus
}
#endif

#endif
