// Cache writes (BF16 copy, FP8-E4M3FN, NVFP4) through slot_mapping, and the
// BF16 absmax used for FP8 calibration.
//
// Method: metrale API page "metrale_model_layers/layers/ops/prefill_attn_b.rs",
// reshape_and_cache_nvfp4 (each token's K and V rows go to the page and offset
// its slot names; E2M1 values with one E4M3 scale per 16; one workgroup per
// token) and bf16_absmax (max |x| folded into an f32 with an atomic max).
//
// One workgroup per token (256 lanes, or the whole waves a short row needs).
// A lane moves 16 bytes of BF16 source
// (8 elements) per step; the FP8 path writes 8 code bytes per step and the
// NVFP4 path handles a whole 16-element group (two 16-byte source loads, 8
// code bytes and one scale byte) per step.
#include "../../include/pkd.h"
#include "device_common.hpp"
#include "validate.hpp"

namespace pkd {

struct WriteArgs {
  const uint16_t* key;
  const uint16_t* value;
  uint8_t* k_cache;
  uint8_t* v_cache;
  const int32_t* slots;
  uint32_t num_kv_heads;
  uint32_t head_dim;
  uint32_t block_size;
  uint32_t key_stride;
  uint32_t value_stride;
  float k_scale;
  float v_scale;
  uint64_t page_bytes;      // bytes per page (BF16: bs*Hkv*D*2, FP8: cache_stride, NVFP4: block stride)
  uint64_t data_section;    // NVFP4: offset of the scale section within a page
};

enum Fmt { kBf16 = 0, kFp8 = 1, kNvfp4 = 2 };

template <int FMT>
__device__ __forceinline__ void write_rows(const WriteArgs& a, const uint16_t* src,
                                           uint8_t* cache, float scale, uint64_t row_base_elem,
                                           uint64_t page_base, uint32_t off) {
  const uint32_t D = a.head_dim;
  const uint32_t row = a.num_kv_heads * D;          // elements in one token's row
  if constexpr (FMT == kBf16) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(cache + page_base) + uint64_t(off) * row;
    for (uint32_t c = threadIdx.x; c < row / 8; c += blockDim.x) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(src + row_base_elem + c * 8);
      *reinterpret_cast<u32x4*>(dst + c * 8) = v;
    }
  } else if constexpr (FMT == kFp8) {
    uint8_t* dst = cache + page_base + uint64_t(off) * row;
    for (uint32_t c = threadIdx.x; c < row / 8; c += blockDim.x) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(src + row_base_elem + c * 8);
      *reinterpret_cast<u32x2*>(dst + c * 8) = fp8_encode8(v, scale);
    }
  } else {
    uint8_t* data = cache + page_base + uint64_t(off) * (row / 2);
    uint8_t* scales = cache + page_base + a.data_section + uint64_t(off) * (row / 16);
    for (uint32_t g = threadIdx.x; g < row / 16; g += blockDim.x) {
      const u32x4 v0 = *reinterpret_cast<const u32x4*>(src + row_base_elem + g * 16);
      const u32x4 v1 = *reinterpret_cast<const u32x4*>(src + row_base_elem + g * 16 + 8);
      uint32_t s_code;
      *reinterpret_cast<u32x2*>(data + g * 8) = nvfp4_encode16(v0, v1, s_code);
      scales[g] = uint8_t(s_code);
    }
  }
}

template <int FMT>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(WriteArgs a) {
  const uint32_t t = blockIdx.x;
  const int32_t slot = a.slots[t];
  // Rows that one pass of the workgroup covers (8 elements a lane, 16 for an
  // NVFP4 group): the K and V source loads go out together with the slot load,
  // instead of the slot, then K, then V (the compiler cannot move V's loads
  // above K's stores: the pointers may alias).
  constexpr uint32_t PER = FMT == kNvfp4 ? 16 : 8;
  const uint32_t row = a.num_kv_heads * a.head_dim;
  if (row <= 256 * PER) {
    const uint32_t c = threadIdx.x;
    const bool act = c < row / PER;
    u32x4 k0 = {0u, 0u, 0u, 0u}, v0 = k0, k1 = k0, v1 = k0;
    if (act) {
      const uint16_t* ks = a.key + uint64_t(t) * a.key_stride + c * PER;
      const uint16_t* vs = a.value + uint64_t(t) * a.value_stride + c * PER;
      k0 = *reinterpret_cast<const u32x4*>(ks);
      v0 = *reinterpret_cast<const u32x4*>(vs);
      if constexpr (FMT == kNvfp4) {
        k1 = *reinterpret_cast<const u32x4*>(ks + 8);
        v1 = *reinterpret_cast<const u32x4*>(vs + 8);
      }
    }
    if (slot < 0 || !act) return;
    const uint32_t off = uint32_t(slot) % a.block_size;
    const uint64_t page_base = uint64_t(uint32_t(slot) / a.block_size) * a.page_bytes;
    if constexpr (FMT == kBf16) {
      const uint64_t at = page_base + (uint64_t(off) * row + c * 8) * 2;
      *reinterpret_cast<u32x4*>(a.k_cache + at) = k0;
      *reinterpret_cast<u32x4*>(a.v_cache + at) = v0;
    } else if constexpr (FMT == kFp8) {
      const uint64_t at = page_base + uint64_t(off) * row + c * 8;
      *reinterpret_cast<u32x2*>(a.k_cache + at) = fp8_encode8(k0, a.k_scale);
      *reinterpret_cast<u32x2*>(a.v_cache + at) = fp8_encode8(v0, a.v_scale);
    } else {
      const uint64_t at = page_base + uint64_t(off) * (row / 2) + c * 8;
      const uint64_t sat = page_base + a.data_section + uint64_t(off) * (row / 16) + c;
      uint32_t ks_code, vs_code;
      const u32x2 kc = nvfp4_encode16(k0, k1, ks_code);
      const u32x2 vc = nvfp4_encode16(v0, v1, vs_code);
      *reinterpret_cast<u32x2*>(a.k_cache + at) = kc;
      *reinterpret_cast<u32x2*>(a.v_cache + at) = vc;
      a.k_cache[sat] = uint8_t(ks_code);
      a.v_cache[sat] = uint8_t(vs_code);
    }
    return;
  }
  if (slot < 0) return;
  const uint32_t page = uint32_t(slot) / a.block_size;
  const uint32_t off = uint32_t(slot) % a.block_size;
  const uint64_t page_base = uint64_t(page) * a.page_bytes;
  write_rows<FMT>(a, a.key, a.k_cache, a.k_scale, uint64_t(t) * a.key_stride, page_base, off);
  write_rows<FMT>(a, a.value, a.v_cache, a.v_scale, uint64_t(t) * a.value_stride, page_base, off);
}

// absmax: each lane folds 8 BF16 per 16-byte load over a grid-stride loop,
// the workgroup reduces through LDS, one atomic max per workgroup.
__global__ __launch_bounds__(256) void bf16_absmax_kernel(const uint16_t* data, float* out,
                                                          uint64_t n) {
  float m = 0.0f;
  const uint64_t nvec = n / 8;
  const uint64_t stride = uint64_t(gridDim.x) * blockDim.x;
  for (uint64_t i = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < nvec; i += stride) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(data + i * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = __builtin_fabsf(bf16_lo(v[j]));
      const float hi = __builtin_fabsf(bf16_hi(v[j]));
      if (lo == lo) m = fmaxf(m, lo);          // NaN compares unequal: skipped
      if (hi == hi) m = fmaxf(m, hi);
    }
  }
  if (blockIdx.x == 0) {                          // tail elements past the last full vector
    for (uint64_t i = nvec * 8 + threadIdx.x; i < n; i += blockDim.x) {
      const float x = __builtin_fabsf(__uint_as_float(uint32_t(data[i]) << 16));
      if (x == x) m = fmaxf(m, x);
    }
  }
  m = wave_max(m);
  __shared__ float part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
    // non-negative floats order like their bit patterns
    atomicMax(reinterpret_cast<unsigned int*>(out), __float_as_uint(m));
  }
}

static int launch_status() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? kOk : kLaunch;
}

// One workgroup per token: 256 lanes, or for a row that one pass covers,
// just the whole waves that row needs (an NVFP4 row of 1024 values is 64
// groups: one wave), so no lane idles and more tokens are resident per CU.
template <int FMT>
static int launch_write(const WriteArgs& a, uint32_t num_tokens, hipStream_t stream) {
  constexpr uint32_t per = FMT == kNvfp4 ? 16 : 8;
  const uint32_t units = a.num_kv_heads * a.head_dim / per;
  const uint32_t nt = units <= 256 ? (units + 63) / 64 * 64 : 256;
  hipLaunchKernelGGL(reshape_and_cache_kernel<FMT>, dim3(num_tokens), dim3(nt), 0, stream, a);
  return launch_status();
}

}  // namespace pkd

using namespace pkd;

extern "C" PKD_API int reshape_and_cache_bf16(const uint16_t* key, const uint16_t* value,
                                              uint16_t* k_cache, uint16_t* v_cache,
                                              const int32_t* slot_mapping, uint32_t num_tokens,
                                              uint32_t num_kv_heads, uint32_t head_dim,
                                              uint32_t block_size, uint32_t key_stride,
                                              uint32_t value_stride, hipStream_t stream) {
  if (num_tokens == 0) return kOk;
  int st = check_cache_write(key, value, k_cache, v_cache, slot_mapping, num_kv_heads, head_dim,
                             block_size, key_stride, value_stride);
  if (st) return st;
  WriteArgs a{key, value, reinterpret_cast<uint8_t*>(k_cache), reinterpret_cast<uint8_t*>(v_cache),
              slot_mapping, num_kv_heads, head_dim, block_size, key_stride, value_stride,
              1.0f, 1.0f, uint64_t(block_size) * num_kv_heads * head_dim * 2, 0};
  return launch_write<kBf16>(a, num_tokens, stream);
}

extern "C" PKD_API int reshape_and_cache_fp8(const uint16_t* key, const uint16_t* value,
                                             uint8_t* k_cache, uint8_t* v_cache,
                                             const int32_t* slot_mapping, uint32_t num_tokens,
                                             uint32_t num_kv_heads, uint32_t head_dim,
                                             uint32_t block_size, uint32_t key_stride,
                                             uint32_t value_stride, float k_scale, float v_scale,
                                             uint64_t cache_stride, hipStream_t stream) {
  if (num_tokens == 0) return kOk;
  int st = check_cache_write(key, value, k_cache, v_cache, slot_mapping, num_kv_heads, head_dim,
                             block_size, key_stride, value_stride);
  if (st) return st;
  st = check_fp8_stride(num_kv_heads, head_dim, block_size, cache_stride);
  if (st) return st;
  WriteArgs a{key, value, k_cache, v_cache, slot_mapping, num_kv_heads, head_dim, block_size,
              key_stride, value_stride, k_scale, v_scale, cache_stride, 0};
  return launch_write<kFp8>(a, num_tokens, stream);
}

extern "C" PKD_API int reshape_and_cache_nvfp4(const uint16_t* key, const uint16_t* value,
                                               uint8_t* k_cache, uint8_t* v_cache,
                                               const int32_t* slot_mapping, uint32_t num_tokens,
                                               uint32_t num_kv_heads, uint32_t head_dim,
                                               uint32_t block_size, uint32_t key_stride,
                                               uint32_t value_stride, uint64_t block_stride_bytes,
                                               uint64_t data_section_bytes, hipStream_t stream) {
  if (num_tokens == 0) return kOk;
  int st = check_cache_write(key, value, k_cache, v_cache, slot_mapping, num_kv_heads, head_dim,
                             block_size, key_stride, value_stride);
  if (st) return st;
  st = check_nvfp4_sections(num_kv_heads, head_dim, block_size, block_stride_bytes,
                            data_section_bytes);
  if (st) return st;
  WriteArgs a{key, value, k_cache, v_cache, slot_mapping, num_kv_heads, head_dim, block_size,
              key_stride, value_stride, 1.0f, 1.0f, block_stride_bytes, data_section_bytes};
  return launch_write<kNvfp4>(a, num_tokens, stream);
}

extern "C" PKD_API int bf16_absmax(const uint16_t* data, float* out_max, uint64_t n_elems,
                                   hipStream_t stream) {
  if (n_elems == 0) return kOk;
  if (!data || !out_max || !aligned16(data) || (reinterpret_cast<uintptr_t>(out_max) & 3u))
    return kInvalid;
  const uint64_t per_block = 256ull * 8 * 8;      // 8 vector loads per lane at least
  uint64_t blocks = (n_elems + per_block - 1) / per_block;
  if (blocks > 2048) blocks = 2048;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(bf16_absmax_kernel, dim3(uint32_t(blocks)), dim3(256), 0, stream, data,
                     out_max, n_elems);
  return launch_status();
}
