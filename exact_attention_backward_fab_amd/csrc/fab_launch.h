// fab_launch.h -- host-side launch interface between the C ABI (fab_api.cpp)
// and the kernels (fab_kernels.hip).  Internal to libfab.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fab {

struct Dims {
    int B, H, Hkv, N, M, DK, DV;
};

// Padded head dimensions the kernels are instantiated for.
int padded_dim(int d);                 // 32, 64, 128 or 192; 0 if unsupported
bool bwd_supported(int dkp, int dvp, int bf16);

// Block map of the additive mask: u8 [ceil(N/32)][ceil(M/32)].
hipError_t launch_block_map(const uint16_t *mask, uint8_t *map, const Dims &d, hipStream_t s);

// Forward with row log-sum-exp (natural log, -inf for all-masked rows).
hipError_t launch_forward(const float *q, const float *k, const float *v, const uint16_t *mask,
                          const uint8_t *map, float scale, int bf16, float *O, float *lse,
                          const Dims &d, hipStream_t s);

// Delta = rowsum(d o O) [N,H,B]; zero the dQ slice [0, nq) and the blob pads.
hipError_t launch_prep(const float *dO, const float *O, float *delta, float *blob, int64_t nq,
                       int64_t off_k, int64_t nk, int64_t off_v, int64_t nv, int64_t total,
                       const Dims &d, hipStream_t s);

// KV-block-outer backward: dV, dK per key tile (stored into dk/dv with
// per-query-head layout when part_heads != 0), dQ by f32 atomics into dq.
hipError_t launch_backward(const float *q, const float *k, const float *v, const float *dO,
                           const uint16_t *mask, const uint8_t *map, const float *lse,
                           const float *delta, float scale, int bf16, float *dq, float *dk,
                           float *dv, int part_heads, const Dims &d, hipStream_t s);

// dst[c, m, g, b] = sum_{r < rk2} part[c, m, g*rk2 + r, b] for one of dK / dV.
hipError_t launch_gqa_reduce(const float *part, float *dst, int D, const Dims &d, hipStream_t s);

// Fill n floats with zero.
hipError_t launch_zero(float *p, int64_t n, hipStream_t s);

}  // namespace fab
