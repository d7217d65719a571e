// Device-side packer: interchange format -> slot layout (see common.h).
// MOE_WF_Q4_G32: one thread per (tile, 32-element group): 8 rows x 16 bytes of
// nibbles (turned from offset binary into two's complement by flipping each
// nibble's top bit) and the 8 fp16 scales of that group.
#include "common.h"

namespace moe {
namespace {

__device__ inline uint4 to_twos(uint4 v) {
  return make_uint4(v.x ^ 0x88888888u, v.y ^ 0x88888888u, v.z ^ 0x88888888u, v.w ^ 0x88888888u);
}

__global__ __launch_bounds__(256) void k_pack(int H, int I, const uint8_t *qg, const uint16_t *sg, const uint8_t *qu,
                                              const uint16_t *su, const uint8_t *qd, const uint16_t *sd, uint8_t *dst) {
  const long id = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long ngh = H / kGroup, ngi = I / kGroup;
  const long n_gu = (long)(I / kGuPairs) * ngh;
  const long n_dn = (long)(H / kDnRows) * ngi;
  if (id < n_gu) {
    const int t = (int)(id / ngh), g = (int)(id - (long)t * ngh);
    uint8_t *tile = dst + (size_t)t * gu_tile_bytes(H, kWfQ4G32);
    uint16_t *scl = (uint16_t *)(tile + (size_t)kGuRows * (H / 2));
    for (int i = 0; i < kGuRows; ++i) {
      const int r = kGuPairs * t + i / 2;
      const uint8_t *q = (i & 1) ? qu : qg;
      const uint16_t *s = (i & 1) ? su : sg;
      *(uint4 *)(tile + (size_t)i * (H / 2) + g * 16) = to_twos(*(const uint4 *)(q + (size_t)r * (H / 2) + g * 16));
      scl[g * kGuRows + i] = s[(size_t)r * ngh + g];
    }
  } else if (id < n_gu + n_dn) {
    const long j = id - n_gu;
    const int t = (int)(j / ngi), g = (int)(j - (long)t * ngi);
    uint8_t *tile = dst + down_offset(H, I, kWfQ4G32) + (size_t)t * dn_tile_bytes(I, kWfQ4G32);
    uint16_t *scl = (uint16_t *)(tile + (size_t)kDnRows * (I / 2));
    for (int i = 0; i < kDnRows; ++i) {
      const int r = kDnRows * t + i;
      *(uint4 *)(tile + (size_t)i * (I / 2) + g * 16) = to_twos(*(const uint4 *)(qd + (size_t)r * (I / 2) + g * 16));
      scl[g * kDnRows + i] = sd[(size_t)r * ngi + g];
    }
  }
}

// Row-scaled formats: one thread per (tile, 32-element group) copies the 8
// rows' bytes of that group (int4 nibbles flipped to two's complement; int8 bytes
// as they are); the group-0 thread also writes the tile's 8 fp32 row scales.
template <int WF>
__global__ __launch_bounds__(256) void k_pack_rows(int H, int I, const uint8_t *qg, const float *sg,
                                                   const uint8_t *qu, const float *su, const uint8_t *qd,
                                                   const float *sd, uint8_t *dst) {
  constexpr int GB = group_bytes(WF);
  const long id = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long ngh = H / kGroup, ngi = I / kGroup;
  const long n_gu = (long)(I / kGuPairs) * ngh;
  const long n_dn = (long)(H / kDnRows) * ngi;
  auto copy_group = [&](uint8_t *d, const uint8_t *q) {
#pragma unroll
    for (int b = 0; b < GB; b += 16) {
      const uint4 v = *(const uint4 *)(q + b);
      *(uint4 *)(d + b) = WF == kWfQ8Row ? v : to_twos(v);
    }
  };
  if (id < n_gu) {
    const int t = (int)(id / ngh), g = (int)(id - (long)t * ngh);
    const int64_t rb = row_bytes(H, WF);
    uint8_t *tile = dst + (size_t)t * gu_tile_bytes(H, WF);
    float *scl = (float *)(tile + (size_t)kGuRows * rb);
    for (int i = 0; i < kGuRows; ++i) {
      const int r = kGuPairs * t + i / 2;
      copy_group(tile + (size_t)i * rb + g * GB, ((i & 1) ? qu : qg) + (size_t)r * rb + g * GB);
      if (g == 0) scl[i] = ((i & 1) ? su : sg)[r];
    }
  } else if (id < n_gu + n_dn) {
    const long j = id - n_gu;
    const int t = (int)(j / ngi), g = (int)(j - (long)t * ngi);
    const int64_t rb = row_bytes(I, WF);
    uint8_t *tile = dst + down_offset(H, I, WF) + (size_t)t * dn_tile_bytes(I, WF);
    float *scl = (float *)(tile + (size_t)kDnRows * rb);
    for (int i = 0; i < kDnRows; ++i) {
      const int r = kDnRows * t + i;
      copy_group(tile + (size_t)i * rb + g * GB, qd + (size_t)r * rb + g * GB);
      if (g == 0) scl[i] = sd[r];
    }
  }
}

}  // namespace

hipError_t launch_pack_rows(int H, int I, int wf, const uint8_t *qg, const float *sg, const uint8_t *qu,
                            const float *su, const uint8_t *qd, const float *sd, uint8_t *dst, hipStream_t st) {
  const long n = (long)(I / kGuPairs) * (H / kGroup) + (long)(H / kDnRows) * (I / kGroup);
  const dim3 g((unsigned)((n + 255) / 256)), b(256);
  if (wf == kWfQ8Row) MOE_LAUNCH(k_pack_rows<kWfQ8Row>, g, b, 0, st, H, I, qg, sg, qu, su, qd, sd, dst);
  else MOE_LAUNCH(k_pack_rows<kWfQ4Row>, g, b, 0, st, H, I, qg, sg, qu, su, qd, sd, dst);
  return hipGetLastError();
}

hipError_t launch_pack(int H, int I, const uint8_t *qg, const uint16_t *sg, const uint8_t *qu, const uint16_t *su,
                       const uint8_t *qd, const uint16_t *sd, uint8_t *dst, hipStream_t st) {
  const long n = (long)(I / kGuPairs) * (H / kGroup) + (long)(H / kDnRows) * (I / kGroup);
  MOE_LAUNCH(k_pack, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, H, I, qg, sg, qu, su, qd, sd, dst);
  return hipGetLastError();
}

}  // namespace moe
