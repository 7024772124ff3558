// Cache writes on gfx950: storing new tokens' K/V into their paged slots, and
// the copy-on-write block copies.
//
// Storing a token follows the append_token store into cache[block, slot] of
// the PagedAttentionManager listing (youngju.dev "vLLM inference
// optimization", PagedAttention section); the copy is the copy-on-write of a
// shared block that diverges (media.tcdigital.jp, "memory sharing for
// parallel sampling").  Both are bit copies.
//
// Pool layout (see include/pa.h): [N][H][tile], tiles in MFMA operand order
// (k_tile_off / v_tile_off; FP8 pools k8_tile_off / v8_tile_off).
//
// FP8 pools (ta-paperlens "in practice": a smaller KV data type as a serving
// setting) store OCP E4M3 codes with one scale per pool.
//
// Also here: the one-launch staging copy of a step's metadata from pinned
// host memory (pa_stage_copy).
#include "pa_device.h"

namespace pa {

// One thread per (token, kv head, 8-dim chunk): the 8 K values are contiguous
// in the tile (one 16-byte store); the 8 V values land 8 elements apart.
template <int D>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const f16* __restrict__ k, const f16* __restrict__ v, const int32_t* __restrict__ slots,
    int32_t num_tokens, int32_t n_kv, int32_t num_blocks, f16* __restrict__ kp,
    f16* __restrict__ vp) {
  constexpr int kChunks = D / 8;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = static_cast<int64_t>(num_tokens) * n_kv * kChunks;
  if (idx >= total) return;
  const int chunk = static_cast<int>(idx % kChunks);
  const int64_t th = idx / kChunks;
  const int h = static_cast<int>(th % n_kv);
  const int64_t t = th / n_kv;
  const int32_t s = slots[t];
  if (s < 0 || s >= num_blocks * kBlock) return;
  const int64_t blk = s / kBlock;
  const int off = s % kBlock;
  const int64_t src = (t * n_kv + h) * D + chunk * 8;
  const f16x8 kv = *reinterpret_cast<const f16x8*>(k + src);
  const f16x8 vv = *reinterpret_cast<const f16x8*>(v + src);
  const int64_t tile = (blk * n_kv + h) * (kBlock * D);
  *reinterpret_cast<f16x8*>(kp + tile + k_tile_off(off, chunk * 8)) = kv;
  f16* vt = vp + tile + v_tile_off(off, chunk * 8);
#pragma unroll
  for (int e = 0; e < 8; ++e) vt[e * 8] = vv[e];  // dims chunk*8 + e: same 16-dim half
}

// One workgroup per (copy, kv head): slots [0, n) of the K and V tiles, as
// 16-byte K chunks and single V elements.
template <int D>
__global__ __launch_bounds__(256) void copy_blocks_kernel(const pa_copy* __restrict__ copies,
                                                          int32_t n_kv, int32_t num_blocks,
                                                          f16* __restrict__ kp,
                                                          f16* __restrict__ vp) {
  const pa_copy c = copies[blockIdx.x];
  const int h = blockIdx.y;
  if (c.src < 0 || c.src >= num_blocks || c.dst < 0 || c.dst >= num_blocks) return;
  if (c.n_slots <= 0 || c.n_slots > kBlock || c.src == c.dst) return;
  const int n = c.n_slots;
  const int64_t st = (static_cast<int64_t>(c.src) * n_kv + h) * (kBlock * D);
  const int64_t dt = (static_cast<int64_t>(c.dst) * n_kv + h) * (kBlock * D);
  for (int i = threadIdx.x; i < n * (D / 8); i += blockDim.x) {
    const int off = k_tile_off(i % n, (i / n) * 8);
    *reinterpret_cast<f16x8*>(kp + dt + off) = *reinterpret_cast<const f16x8*>(kp + st + off);
  }
  for (int i = threadIdx.x; i < n * D; i += blockDim.x) {
    const int off = v_tile_off(i % n, i / n);
    vp[dt + off] = vp[st + off];
  }
}

// FP8 pools: the value times the fp32 reciprocal of the pool's scale, clamped
// to the E4M3 range by comparisons (so NaN passes through), converted with
// round-to-nearest-even.  Two values go into the low (hi = false) or high
// 16 bits of `w`, first value in the lower byte.
__device__ __forceinline__ float clamp_e4m3(float x) {
  return x > 448.0f ? 448.0f : (x < -448.0f ? -448.0f : x);
}
template <bool HI>
__device__ __forceinline__ uint32_t pack_e4m3x2(f16 a, f16 b, float inv, uint32_t w) {
  const float x = clamp_e4m3(static_cast<float>(a) * inv);
  const float y = clamp_e4m3(static_cast<float>(b) * inv);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(x, y, static_cast<int>(w), HI));
}
// Eight values as eight codes, element e in byte e.
__device__ __forceinline__ uint2 quantize8(f16x8 v, float inv) {
  uint2 r;
  r.x = pack_e4m3x2<false>(v[0], v[1], inv, 0u);
  r.x = pack_e4m3x2<true>(v[2], v[3], inv, r.x);
  r.y = pack_e4m3x2<false>(v[4], v[5], inv, 0u);
  r.y = pack_e4m3x2<true>(v[6], v[7], inv, r.y);
  return r;
}

// The fp16 kernel's thread mapping: the 8 K codes of a chunk are contiguous
// in the FP8 tile (one 8-byte store); the 8 V codes land 16 bytes apart.
template <int D>
__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(
    const f16* __restrict__ k, const f16* __restrict__ v, const int32_t* __restrict__ slots,
    int32_t num_tokens, int32_t n_kv, int32_t num_blocks, float k_inv, float v_inv,
    uint8_t* __restrict__ kp, uint8_t* __restrict__ vp) {
  constexpr int kChunks = D / 8;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = static_cast<int64_t>(num_tokens) * n_kv * kChunks;
  if (idx >= total) return;
  const int chunk = static_cast<int>(idx % kChunks);
  const int64_t th = idx / kChunks;
  const int h = static_cast<int>(th % n_kv);
  const int64_t t = th / n_kv;
  const int32_t s = slots[t];
  if (s < 0 || s >= num_blocks * kBlock) return;
  const int64_t blk = s / kBlock;
  const int off = s % kBlock;
  const int64_t src = (t * n_kv + h) * D + chunk * 8;
  const uint2 kc = quantize8(*reinterpret_cast<const f16x8*>(k + src), k_inv);
  const uint2 vc = quantize8(*reinterpret_cast<const f16x8*>(v + src), v_inv);
  const int64_t tile = (blk * n_kv + h) * (kBlock * D);
  *reinterpret_cast<uint2*>(kp + tile + k8_tile_off(off, chunk * 8)) = kc;
  uint8_t* vt = vp + tile + v8_tile_off(off, chunk * 8);
#pragma unroll
  for (int e = 0; e < 8; ++e)  // dims chunk*8 + e: same 16-dim half, 16 bytes apart
    vt[e * 16] = static_cast<uint8_t>((e < 4 ? vc.x : vc.y) >> (8 * (e & 3)));
}

// Copy-on-write copy in FP8 pools: slots [0, n) as 8-byte K runs and single
// V bytes.
template <int D>
__global__ __launch_bounds__(256) void copy_blocks_fp8_kernel(const pa_copy* __restrict__ copies,
                                                              int32_t n_kv, int32_t num_blocks,
                                                              uint8_t* __restrict__ kp,
                                                              uint8_t* __restrict__ vp) {
  const pa_copy c = copies[blockIdx.x];
  const int h = blockIdx.y;
  if (c.src < 0 || c.src >= num_blocks || c.dst < 0 || c.dst >= num_blocks) return;
  if (c.n_slots <= 0 || c.n_slots > kBlock || c.src == c.dst) return;
  const int n = c.n_slots;
  const int64_t st = (static_cast<int64_t>(c.src) * n_kv + h) * (kBlock * D);
  const int64_t dt = (static_cast<int64_t>(c.dst) * n_kv + h) * (kBlock * D);
  for (int i = threadIdx.x; i < n * (D / 8); i += blockDim.x) {
    const int off = k8_tile_off(i % n, (i / n) * 8);
    *reinterpret_cast<uint2*>(kp + dt + off) = *reinterpret_cast<const uint2*>(kp + st + off);
  }
  for (int i = threadIdx.x; i < n * D; i += blockDim.x) {
    const int off = v8_tile_off(i % n, i / n);
    vp[dt + off] = vp[st + off];
  }
}

static bool valid_view(const pa_kv_view& kv) {
  return kv.k_pool != nullptr && kv.v_pool != nullptr && kv.num_blocks > 0 &&
         static_cast<int64_t>(kv.num_blocks) * kBlock < (1LL << 31) &&
         kv.block_size == kBlock && kv.num_kv_heads > 0 &&
         (kv.head_dim == 64 || kv.head_dim == 128) && aligned16(kv.k_pool) &&
         aligned16(kv.v_pool);
}

static bool valid_scale(float x) { return x > 0.0f && x <= 3.0e38f; }

static bool valid_view(const pa_kv_view_fp8& kv) {
  return kv.k_pool != nullptr && kv.v_pool != nullptr && kv.num_blocks > 0 &&
         static_cast<int64_t>(kv.num_blocks) * kBlock < (1LL << 31) &&
         kv.block_size == kBlock && kv.num_kv_heads > 0 &&
         (kv.head_dim == 64 || kv.head_dim == 128) && aligned16(kv.k_pool) &&
         aligned16(kv.v_pool) && valid_scale(kv.k_scale) && valid_scale(kv.v_scale);
}


// Whole tiles between the pools and a contiguous buffer [n][n_kv][tile] in
// the pools' own tile order, for moving a preempted sequence's blocks out
// of the pool and back (GATHER: pool -> buffer, else buffer -> pool).  One
// workgroup per (entry, kv head), 16-byte chunks; entries outside
// [0, num_blocks) are skipped.
template <bool GATHER>
__global__ __launch_bounds__(256) void block_transfer_kernel(
    const int32_t* __restrict__ blocks, int32_t n_kv, int32_t num_blocks, int32_t tile_chunks,
    u32x4* __restrict__ kp, u32x4* __restrict__ vp, u32x4* __restrict__ kb,
    u32x4* __restrict__ vb) {
  const int32_t b = blocks[blockIdx.x];
  if (b < 0 || b >= num_blocks) return;
  const int h = blockIdx.y;
  const int64_t po = (static_cast<int64_t>(b) * n_kv + h) * tile_chunks;
  const int64_t bo = (static_cast<int64_t>(blockIdx.x) * n_kv + h) * tile_chunks;
  for (int c = threadIdx.x; c < tile_chunks; c += blockDim.x) {
    if (GATHER) {
      kb[bo + c] = kp[po + c];
      vb[bo + c] = vp[po + c];
    } else {
      kp[po + c] = kb[bo + c];
      vp[po + c] = vb[bo + c];
    }
  }
}

static pa_status block_transfer(bool gather, const int32_t* blocks, int32_t n, void* k_pool,
                                void* v_pool, int32_t num_blocks, int32_t block_size,
                                int32_t n_kv, int32_t head_dim, int32_t elem_bytes, void* k_buf,
                                void* v_buf, void* stream) {
  if (k_pool == nullptr || v_pool == nullptr || block_size != kBlock || num_blocks <= 0 ||
      n_kv <= 0 || n_kv > 65535 || (head_dim != 64 && head_dim != 128) || n < 0)
    return PA_ERR_INVALID;
  if (n == 0) return PA_OK;
  if (blocks == nullptr || k_buf == nullptr || v_buf == nullptr || !aligned16(k_buf) ||
      !aligned16(v_buf) || !aligned16(k_pool) || !aligned16(v_pool))
    return PA_ERR_INVALID;
  const int32_t chunks = head_dim * elem_bytes;  // 16 * D * elem_bytes / 16
  const dim3 grid(static_cast<uint32_t>(n), static_cast<uint32_t>(n_kv));
  hipStream_t s = static_cast<hipStream_t>(stream);
  u32x4* kp = static_cast<u32x4*>(k_pool);
  u32x4* vp = static_cast<u32x4*>(v_pool);
  u32x4* kb = static_cast<u32x4*>(k_buf);
  u32x4* vb = static_cast<u32x4*>(v_buf);
  if (gather)
    block_transfer_kernel<true><<<grid, dim3(256), 0, s>>>(blocks, n_kv, num_blocks, chunks, kp,
                                                           vp, kb, vb);
  else
    block_transfer_kernel<false><<<grid, dim3(256), 0, s>>>(blocks, n_kv, num_blocks, chunks, kp,
                                                            vp, kb, vb);
  return launch_status();
}

}  // namespace pa

using namespace pa;

extern "C" pa_status pa_reshape_and_cache(const pa_half* k, const pa_half* v,
                                          const int32_t* slot_mapping, int32_t num_tokens,
                                          pa_kv_view kv, void* stream) {
  if (!valid_view(kv) || num_tokens < 0) return PA_ERR_INVALID;
  if (num_tokens == 0) return PA_OK;
  if (k == nullptr || v == nullptr || slot_mapping == nullptr || !aligned16(k) || !aligned16(v))
    return PA_ERR_INVALID;
  const int64_t total = static_cast<int64_t>(num_tokens) * kv.num_kv_heads * (kv.head_dim / 8);
  const int64_t blocks = (total + 255) / 256;
  if (blocks > INT32_MAX) return PA_ERR_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const f16* kk = reinterpret_cast<const f16*>(k);
  const f16* vv = reinterpret_cast<const f16*>(v);
  f16* kp = reinterpret_cast<f16*>(kv.k_pool);
  f16* vp = reinterpret_cast<f16*>(kv.v_pool);
  if (kv.head_dim == 128)
    reshape_and_cache_kernel<128><<<dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s>>>(
        kk, vv, slot_mapping, num_tokens, kv.num_kv_heads, kv.num_blocks, kp, vp);
  else
    reshape_and_cache_kernel<64><<<dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s>>>(
        kk, vv, slot_mapping, num_tokens, kv.num_kv_heads, kv.num_blocks, kp, vp);
  return launch_status();
}

extern "C" pa_status pa_copy_blocks(const pa_copy* copies, int32_t n, pa_kv_view kv,
                                    void* stream) {
  if (!valid_view(kv) || n < 0) return PA_ERR_INVALID;
  if (n == 0) return PA_OK;
  if (copies == nullptr || kv.num_kv_heads > 65535) return PA_ERR_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  f16* kp = reinterpret_cast<f16*>(kv.k_pool);
  f16* vp = reinterpret_cast<f16*>(kv.v_pool);
  const dim3 grid(static_cast<uint32_t>(n), static_cast<uint32_t>(kv.num_kv_heads));
  if (kv.head_dim == 128)
    copy_blocks_kernel<128><<<grid, dim3(256), 0, s>>>(copies, kv.num_kv_heads, kv.num_blocks,
                                                       kp, vp);
  else
    copy_blocks_kernel<64><<<grid, dim3(256), 0, s>>>(copies, kv.num_kv_heads, kv.num_blocks,
                                                      kp, vp);
  return launch_status();
}

extern "C" pa_status pa_reshape_and_cache_fp8(const pa_half* k, const pa_half* v,
                                              const int32_t* slot_mapping, int32_t num_tokens,
                                              pa_kv_view_fp8 kv, void* stream) {
  if (!valid_view(kv) || num_tokens < 0) return PA_ERR_INVALID;
  if (num_tokens == 0) return PA_OK;
  if (k == nullptr || v == nullptr || slot_mapping == nullptr || !aligned16(k) || !aligned16(v))
    return PA_ERR_INVALID;
  const int64_t total = static_cast<int64_t>(num_tokens) * kv.num_kv_heads * (kv.head_dim / 8);
  const int64_t blocks = (total + 255) / 256;
  if (blocks > INT32_MAX) return PA_ERR_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const f16* kk = reinterpret_cast<const f16*>(k);
  const f16* vv = reinterpret_cast<const f16*>(v);
  const float k_inv = 1.0f / kv.k_scale;  // fp32, once per call
  const float v_inv = 1.0f / kv.v_scale;
  if (kv.head_dim == 128)
    reshape_and_cache_fp8_kernel<128><<<dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s>>>(
        kk, vv, slot_mapping, num_tokens, kv.num_kv_heads, kv.num_blocks, k_inv, v_inv,
        kv.k_pool, kv.v_pool);
  else
    reshape_and_cache_fp8_kernel<64><<<dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s>>>(
        kk, vv, slot_mapping, num_tokens, kv.num_kv_heads, kv.num_blocks, k_inv, v_inv,
        kv.k_pool, kv.v_pool);
  return launch_status();
}

extern "C" pa_status pa_copy_blocks_fp8(const pa_copy* copies, int32_t n, pa_kv_view_fp8 kv,
                                        void* stream) {
  if (!valid_view(kv) || n < 0) return PA_ERR_INVALID;
  if (n == 0) return PA_OK;
  if (copies == nullptr || kv.num_kv_heads > 65535) return PA_ERR_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<uint32_t>(n), static_cast<uint32_t>(kv.num_kv_heads));
  if (kv.head_dim == 128)
    copy_blocks_fp8_kernel<128><<<grid, dim3(256), 0, s>>>(copies, kv.num_kv_heads,
                                                           kv.num_blocks, kv.k_pool, kv.v_pool);
  else
    copy_blocks_fp8_kernel<64><<<grid, dim3(256), 0, s>>>(copies, kv.num_kv_heads,
                                                          kv.num_blocks, kv.k_pool, kv.v_pool);
  return launch_status();
}

extern "C" pa_status pa_gather_blocks(const int32_t* blocks, int32_t n, pa_kv_view kv,
                                      pa_half* k_out, pa_half* v_out, void* stream) {
  return block_transfer(true, blocks, n, kv.k_pool, kv.v_pool, kv.num_blocks, kv.block_size,
                        kv.num_kv_heads, kv.head_dim, 2, k_out, v_out, stream);
}

extern "C" pa_status pa_scatter_blocks(const int32_t* blocks, int32_t n, pa_kv_view kv,
                                       const pa_half* k_in, const pa_half* v_in, void* stream) {
  return block_transfer(false, blocks, n, kv.k_pool, kv.v_pool, kv.num_blocks, kv.block_size,
                        kv.num_kv_heads, kv.head_dim, 2, const_cast<pa_half*>(k_in),
                        const_cast<pa_half*>(v_in), stream);
}

extern "C" pa_status pa_gather_blocks_fp8(const int32_t* blocks, int32_t n, pa_kv_view_fp8 kv,
                                          uint8_t* k_out, uint8_t* v_out, void* stream) {
  return block_transfer(true, blocks, n, kv.k_pool, kv.v_pool, kv.num_blocks, kv.block_size,
                        kv.num_kv_heads, kv.head_dim, 1, k_out, v_out, stream);
}

extern "C" pa_status pa_scatter_blocks_fp8(const int32_t* blocks, int32_t n, pa_kv_view_fp8 kv,
                                           const uint8_t* k_in, const uint8_t* v_in,
                                           void* stream) {
  return block_transfer(false, blocks, n, kv.k_pool, kv.v_pool, kv.num_blocks, kv.block_size,
                        kv.num_kv_heads, kv.head_dim, 1, const_cast<uint8_t*>(k_in),
                        const_cast<uint8_t*>(v_in), stream);
}

extern "C" pa_status pa_host_device_pointer(const void* host, void** device) {
  if (host == nullptr || device == nullptr) return PA_ERR_INVALID;
  void* d = nullptr;
  if (hipHostGetDevicePointer(&d, const_cast<void*>(host), 0) != hipSuccess || d == nullptr) {
    (void)hipGetLastError();  // not pinned: clear the runtime's sticky error
    return PA_ERR_INVALID;
  }
  *device = d;
  return PA_OK;
}

namespace pa {

// 16-byte chunks, grid-stride; the source is usually pinned host memory read
// across the host link once, hence the non-temporal loads
__global__ __launch_bounds__(256) void stage_copy_kernel(const u32x4* __restrict__ src,
                                                         u32x4* __restrict__ dst, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = __builtin_nontemporal_load(src + i);
}

}  // namespace pa

namespace pa {

typedef int32_t i32x2 __attribute__((ext_vector_type(2)));

// The staging copy plus word updates: threads below n copy 16-byte chunks
// as stage_copy_kernel does; update j (an (index, value) int32 pair) is
// applied by thread j, target[index] = value when the index is in range.
__global__ __launch_bounds__(256) void stage_update_kernel(const u32x4* __restrict__ src,
                                                           u32x4* __restrict__ dst, int64_t n,
                                                           const i32x2* __restrict__ updates,
                                                           int64_t n_updates,
                                                           int32_t* __restrict__ target,
                                                           int64_t target_len) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  for (int64_t i = t0; i < n; i += stride) dst[i] = __builtin_nontemporal_load(src + i);
  for (int64_t j = t0; j < n_updates; j += stride) {
    const i32x2 u = __builtin_nontemporal_load(updates + j);
    if (u[0] >= 0 && u[0] < target_len) target[u[0]] = u[1];
  }
}

}  // namespace pa

extern "C" pa_status pa_stage_copy(const void* src, void* dst, uint64_t bytes, void* stream) {
  if (src == nullptr || dst == nullptr) return PA_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst) | bytes) & 15u)
    return PA_ERR_INVALID;
  const int64_t n = static_cast<int64_t>(bytes / 16);
  if (n == 0) return PA_OK;
  const int64_t wgs = n < 256 * 256 ? (n + 255) / 256 : 256;
  pa::stage_copy_kernel<<<dim3(static_cast<uint32_t>(wgs)), dim3(256), 0,
                          static_cast<hipStream_t>(stream)>>>(
      reinterpret_cast<const pa::u32x4*>(src), reinterpret_cast<pa::u32x4*>(dst), n);
  return pa::launch_status();
}

extern "C" pa_status pa_stage_update(const void* src, void* dst, uint64_t bytes,
                                     const int32_t* updates, int64_t n_updates, int32_t* target,
                                     int64_t target_len, void* stream) {
  if (n_updates < 0 || target_len < 0 || target_len > INT32_MAX) return PA_ERR_INVALID;
  if (bytes > 0 && (src == nullptr || dst == nullptr)) return PA_ERR_INVALID;
  if (n_updates > 0 && (updates == nullptr || target == nullptr)) return PA_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst) | bytes) & 15u)
    return PA_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(updates) & 7u) || (reinterpret_cast<uintptr_t>(target) & 3u))
    return PA_ERR_INVALID;
  const int64_t n = static_cast<int64_t>(bytes / 16);
  const int64_t work = n > n_updates ? n : n_updates;
  if (work == 0) return PA_OK;
  const int64_t wgs = work < 256 * 256 ? (work + 255) / 256 : 256;
  pa::stage_update_kernel<<<dim3(static_cast<uint32_t>(wgs)), dim3(256), 0,
                            static_cast<hipStream_t>(stream)>>>(
      reinterpret_cast<const pa::u32x4*>(src), reinterpret_cast<pa::u32x4*>(dst), n,
      reinterpret_cast<const pa::i32x2*>(updates), n_updates, target, target_len);
  return pa::launch_status();
}

