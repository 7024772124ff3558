// Mixed decode + prefill launch on gfx950.
//
// Mixed step: the decode units of a batch and the tiles of one prefill chunk
// in one launch over one pool (a scheduler step runs both kinds of work in
// one forward pass: ta-paperlens "scheduler skeleton"; techfeed.io ngrok
// summary, "the scheduler").  Workgroups of the prefill launch's size (8
// wavefronts with fp16 pools, 4 with FP8 ones); the first pf_wgs take prefill
// tiles (kv head fastest, then query tile, then key split, as the prefill
// launch's grid), the rest walk the decode work list as the decode launch's
// work-list form does, one walk per wavefront pair (up to 4 or 2 per
// workgroup): as many decode workgroups as stay resident, so that once the
// tiles retire every CU streams K/V with the next unit's loads in flight
// during each unit's epilogue and merged rows buffered in an LDS ring.  The
// prefill tiles, being the long work, start first; decode workgroups fill
// the CUs as tiles retire, so the chunk's ragged end and the launch gap
// between the two kinds of work overlap with memory-bound decode.  Decode
// workgroup j (after the tiles) holds pairs pairs*(j / n_kv) .. of kv head
// j % n_kv, so with 8 kv heads and pf_wgs a multiple of 8 each head's decode
// units land on one XCD, as in the decode launch.
#include <type_traits>

#include "decode_core.h"
#include "prefill_tile.h"

namespace pa {

// Threads of a mixed workgroup: the prefill launch's workgroup size.
template <bool FP8>
constexpr int mixed_threads() {
  return FP8 ? kPfThreads : kPfPPThreads;
}

// LDS of a mixed workgroup (dynamic): one prefill tile's, or the walk state
// of its decode pairs (walk_pair_bytes each), whichever is larger.
template <int D, bool FP8>
constexpr size_t mixed_tile_lds() {
  return FP8 ? sizeof(PrefillLds<D>) : sizeof(PrefillLdsPP<D>);
}

template <int D, bool KEEP, bool FP8>
__global__ __launch_bounds__(mixed_threads<FP8>()) void mixed_step_kernel(
    PrefillArgs pa, int32_t pf_wgs, int32_t pf_qtiles, DecodeArgs da,
    const int32_t* __restrict__ items, int32_t n_items, int32_t pairs, int32_t ring) {
  extern __shared__ f32x4 mixed_lds[];
  const int wg = blockIdx.x;
  if (wg < pf_wgs) {
    const int rest = wg / pa.n_kv;
    // FP8: no raised wave priority here, unlike the prefill launch: tiles
    // that share CUs with decode units starved them (measured on the
    // long-context step: 650 us with the prefill launch's priorities, also
    // when decode units ran at a higher priority, vs 607 us without).  The
    // fp16 tile fills its CU alone (two wavefronts per SIMD at ~211 VGPRs).
    if constexpr (FP8)
      prefill_tile<D, 0, FP8>(pa, wg % pa.n_kv, rest % pf_qtiles, rest / pf_qtiles,
                              *reinterpret_cast<PrefillLds<D>*>(mixed_lds));
    else
      prefill_tile_pp<D>(pa, wg % pa.n_kv, rest % pf_qtiles, rest / pf_qtiles,
                         *reinterpret_cast<PrefillLdsPP<D>*>(mixed_lds));
    return;
  }
  const int G = da.G;
  char* const base = reinterpret_cast<char*>(mixed_lds);
  const size_t pair_bytes = walk_pair_bytes(G, D, ring);
  if (static_cast<int>(threadIdx.x) < pairs) {
    const WalkLds w = walk_carve<D>(base + threadIdx.x * pair_bytes, G, ring);
#pragma unroll
    for (int i = 0; i < kMergeSlots; ++i) {
      w.arrive[i] = 0;
      w.bad[i] = 0;
      w.merged[i] = 0;
    }
    *w.abandon = 0;
  }
  __syncthreads();
  const int pair = uniform(threadIdx.x >> 7);
  if (pair >= pairs) return;
  const int j = wg - pf_wgs;
  const int n_kv = da.n_kv;
  const int g = j % n_kv;
  const int wph = (static_cast<int>(gridDim.x) - pf_wgs) / n_kv * pairs;  // pairs per kv head
  const int y0 = (j / n_kv) * pairs;
  int k_end = 0;  // the most units any pair of this workgroup has
  for (int p = 0; p < pairs; ++p) k_end = max(k_end, walk_units(n_items, wph, y0 + p));
  worklist_walk<D, KEEP, FP8, true>(da, items, n_items, ring, g, y0 + pair, wph, k_end,
                              uniform((threadIdx.x >> 6) & 1), threadIdx.x & 63,
                              walk_carve<D>(base + pair * pair_bytes, G, ring));
}

// Merges after the mixed step's kernel: the prefill (row, head) pairs whose
// key range was split, one wavefront each, in a kernel of their own (the
// decode merge needs ~200 VGPRs, which in one kernel would cut the many short
// prefill merges to 2 wavefronts per SIMD; measured on the long-context
// step: 48 us fused vs 12 + 17 us as two launches), then the decode partitions
// (the decode reduce's code under a name of this file's own).
template <int D>
__global__ __launch_bounds__(kReduceMaxWaves * kWave) void mixed_decode_reduce_kernel(
    DecodeArgs a) {
  decode_reduce_unit<D>(a, blockIdx.x, blockIdx.y);
}

template <int D>
__global__ __launch_bounds__(kWave) void mixed_prefill_reduce_kernel(PrefillArgs pa) {
  prefill_reduce_row<D>(pa.chunk_len, pa.n_kv * pa.G, pa.splits, pa.ws_o, pa.ws_m, pa.ws_l,
                        pa.out, blockIdx.x, blockIdx.y);
}

constexpr uint64_t kMixedWsAlign = 256;

static uint64_t mixed_decode_ws(const pa_decode_batch& d, int32_t num_q_heads, int32_t head_dim) {
  const uint64_t b = pa_decode_workspace_bytes(d.batch, num_q_heads, head_dim, d.max_seq_len,
                                               d.partition_size);
  return (b + kMixedWsAlign - 1) / kMixedWsAlign * kMixedWsAlign;
}

template <int D, bool KEEP, bool FP8>
static const void* step_kernel() {
  return reinterpret_cast<const void*>(&mixed_step_kernel<D, KEEP, FP8>);
}

static const void* pick_step_kernel(int D, bool keep, bool fp8) {
  if (D == 128) {
    if (fp8) return keep ? step_kernel<128, true, true>() : step_kernel<128, false, true>();
    return keep ? step_kernel<128, true, false>() : step_kernel<128, false, false>();
  }
  if (fp8) return keep ? step_kernel<64, true, true>() : step_kernel<64, false, true>();
  return keep ? step_kernel<64, true, false>() : step_kernel<64, false, false>();
}

template <bool KEEP, bool FP8>
static void launch_step(int D, dim3 grid, size_t lds, hipStream_t s, const PrefillArgs& pa,
                        int32_t pf_wgs, int32_t qtiles, const DecodeArgs& da,
                        const int32_t* items, int32_t n_items, int32_t pairs, int32_t ring) {
  const dim3 block(mixed_threads<FP8>());
  if (D == 128)
    mixed_step_kernel<128, KEEP, FP8><<<grid, block, lds, s>>>(pa, pf_wgs, qtiles, da, items,
                                                               n_items, pairs, ring);
  else
    mixed_step_kernel<64, KEEP, FP8><<<grid, block, lds, s>>>(pa, pf_wgs, qtiles, da, items,
                                                              n_items, pairs, ring);
}

// LDS that a mixed workgroup may take: all of a CU's for fp16 pools (the
// tile holds its CU alone), half of it for FP8 ones (two tiles per CU).
constexpr size_t kMixedLdsFp16 = 160 * 1024;
constexpr size_t kMixedLdsFp8 = 80 * 1024;

// Resident mixed workgroups on the current device at this LDS size (CUs
// times the kernel's occupancy), after allowing the kernel that much dynamic
// LDS; both are asked of the runtime once per (device, kernel, LDS size) and
// thread.  0 when the runtime refuses.
static int mixed_resident_wgs(const void* fn, int threads, size_t lds) {
  struct Entry {
    const void* fn;
    size_t lds;
    int dev;
    int wgs;
  };
  thread_local Entry cache[16] = {};
  thread_local int next = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  for (const Entry& e : cache)
    if (e.fn == fn && e.lds == lds && e.dev == dev) return e.wgs;
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                          static_cast<int>(lds)) != hipSuccess)
    return 0;
  int n = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, threads, lds) != hipSuccess || n < 1)
    n = 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 1;
  cache[next] = Entry{fn, lds, dev, n * cus};
  next = (next + 1) % 16;
  return n * cus;
}

// Both pool types: k_pool / v_pool hold fp16 values or (fp8) E4M3 codes with
// one scale per pool, as in the decode and prefill launches.
static pa_status mixed_launch(const pa_decode_batch* dec, const pa_prefill_chunk* pf,
                              const pa_kv_view& kv, bool fp8, float k_scale, float v_scale,
                              int32_t num_q_heads, float scale, void* workspace,
                              uint64_t workspace_bytes, uint32_t flags, void* stream) {
  if (dec == nullptr || pf == nullptr) return PA_ERR_INVALID;
  if (fp8 && !(k_scale > 0.0f && k_scale <= 3.0e38f && v_scale > 0.0f && v_scale <= 3.0e38f))
    return PA_ERR_INVALID;
  if ((flags & ~static_cast<uint32_t>(PA_DECODE_KEEP_KV)) != 0) return PA_ERR_INVALID;
  if (dec->batch > 0 && dec->n_items > 0 && dec->work_items == nullptr) return PA_ERR_INVALID;
  const PoolArgs pool{kv.k_pool, kv.v_pool, kv.num_blocks, kv.block_size, kv.num_kv_heads,
                      kv.head_dim, fp8, fp8 ? k_scale : 1.0f, fp8 ? v_scale : 1.0f};
  const uint64_t dec_ws = mixed_decode_ws(*dec, num_q_heads, kv.head_dim);
  if (workspace_bytes < dec_ws) return PA_ERR_INVALID;
  DecodeArgs da{};
  pa_status st = decode_prepare(dec->out, dec->q, pool, dec->tables, dec->max_blocks,
                                dec->seq_lens, dec->batch, num_q_heads, scale,
                                dec->partition_size, dec->max_seq_len, dec->work_items,
                                dec->n_items, workspace, workspace_bytes, flags, da);
  if (st != PA_OK) return st;
  PrefillArgs pa{};
  dim3 pgrid(0, 0, 0);
  void* pf_ws = workspace == nullptr ? nullptr : static_cast<char*>(workspace) + dec_ws;
  st = prefill_prepare(pf->out, pf->q, kv, pf->table, pf->table_len, pf->q_start, pf->chunk_len,
                       num_q_heads, scale, pf_ws, workspace_bytes - dec_ws, pa, pgrid);
  if (st != PA_OK) return st;
  pa.v_scale = 1.0f;
  if (fp8) {
    pa.kp8 = reinterpret_cast<const uint8_t*>(kv.k_pool);
    pa.vp8 = reinterpret_cast<const uint8_t*>(kv.v_pool);
    pa.kp = pa.vp = nullptr;
    // a score is scale * q . (code * k_scale): k_scale joins the exponent's factor
    pa.scale_log2 *= k_scale;
    pa.v_scale = v_scale;
  }
  // fp16: the prefill launch's 256-M-row tiles (half as many query tiles)
  if (!fp8 && pf->chunk_len > 0)
    pgrid.y = static_cast<uint32_t>((pf->chunk_len + kPfPPMRows / pa.G - 1) / (kPfPPMRows / pa.G));
  const int64_t pf_wgs =
      pf->chunk_len > 0 ? static_cast<int64_t>(pgrid.x) * pgrid.y * pgrid.z : 0;
  const bool keep = (flags & PA_DECODE_KEEP_KV) != 0;
  const int D = kv.head_dim;
  const int threads = fp8 ? mixed_threads<true>() : mixed_threads<false>();
  const size_t tile_lds = fp8 ? (D == 128 ? mixed_tile_lds<128, true>() : mixed_tile_lds<64, true>())
                              : (D == 128 ? mixed_tile_lds<128, false>() : mixed_tile_lds<64, false>());
  // decode walks: one per wavefront pair, with as large a result ring (up to
  // ~16 KiB, at least 2 units) and as many pairs as the LDS allows
  const int32_t n_items = dec->batch > 0 ? dec->n_items : 0;
  int pairs = threads / (kDecodeWaves * kWave);
  const size_t slot = walk_ring_slot_bytes(da.G, D);
  int ring = static_cast<int>(std::max<size_t>(2, kResultRingBytes / slot));
  const size_t budget = fp8 ? kMixedLdsFp8 : kMixedLdsFp16;
  while (ring > 2 && pairs * walk_pair_bytes(da.G, D, ring) > budget) --ring;
  while (pairs > 1 && pairs * walk_pair_bytes(da.G, D, ring) > budget) --pairs;
  const size_t lds =
      std::max(tile_lds, n_items > 0 ? pairs * walk_pair_bytes(da.G, D, ring) : size_t{0});
  if (lds > budget) return PA_ERR_INVALID;  // not reached for G <= 16, D <= 128
  if (pf_wgs == 0 && n_items == 0) return PA_OK;  // nothing to launch
  const int resident = mixed_resident_wgs(pick_step_kernel(D, keep, fp8), threads, lds);
  if (resident < 1) return PA_ERR_HIP;
  // as many decode workgroups as stay resident, a multiple of n_kv, each kv
  // head's pairs no more than its units
  int64_t dec_wgs = 0;
  if (n_items > 0) {
    int64_t per_head = resident / kv.num_kv_heads;
    per_head = std::min<int64_t>(per_head, (n_items + pairs - 1) / pairs);
    per_head = std::max<int64_t>(per_head, 1);
    dec_wgs = per_head * kv.num_kv_heads;
  }
  if (pf_wgs + dec_wgs > 0x7FFFFFFF) return PA_ERR_INVALID;
  if (pf_wgs + dec_wgs == 0) return PA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<uint32_t>(pf_wgs + dec_wgs));
  const int32_t qtiles = static_cast<int32_t>(pgrid.y);
  const int32_t pw = static_cast<int32_t>(pf_wgs);
  if (fp8) {
    if (keep)
      launch_step<true, true>(D, grid, lds, s, pa, pw, qtiles, da, dec->work_items, n_items,
                              pairs, ring);
    else
      launch_step<false, true>(D, grid, lds, s, pa, pw, qtiles, da, dec->work_items, n_items,
                               pairs, ring);
  } else {
    if (keep)
      launch_step<true, false>(D, grid, lds, s, pa, pw, qtiles, da, dec->work_items, n_items,
                               pairs, ring);
    else
      launch_step<false, false>(D, grid, lds, s, pa, pw, qtiles, da, dec->work_items, n_items,
                                pairs, ring);
  }
  if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  if (pf->chunk_len > 0 && pa.splits > 1) {
    const dim3 rgrid(static_cast<uint32_t>(num_q_heads), static_cast<uint32_t>(pf->chunk_len));
    if (D == 128)
      mixed_prefill_reduce_kernel<128><<<rgrid, dim3(kWave), 0, s>>>(pa);
    else
      mixed_prefill_reduce_kernel<64><<<rgrid, dim3(kWave), 0, s>>>(pa);
    if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  }
  if (dec->batch > 0 && da.p_max > 1) {
    const dim3 rgrid(static_cast<uint32_t>(kv.num_kv_heads), static_cast<uint32_t>(dec->batch));
    if (D == 128)
      mixed_decode_reduce_kernel<128><<<rgrid, dim3(reduce_waves(da.p_max) * kWave),
                                 reduce_lds(da.p_max, da.G, 128), s>>>(da);
    else
      mixed_decode_reduce_kernel<64><<<rgrid, dim3(reduce_waves(da.p_max) * kWave),
                                 reduce_lds(da.p_max, da.G, 64), s>>>(da);
  }
  return launch_status();
}

}  // namespace pa

using namespace pa;

extern "C" uint64_t pa_mixed_workspace_bytes(const pa_decode_batch* dec,
                                             const pa_prefill_chunk* pf, int32_t num_q_heads,
                                             int32_t head_dim) {
  if (dec == nullptr || pf == nullptr) return 0;
  return mixed_decode_ws(*dec, num_q_heads, head_dim) +
         prefill_ws_bytes(pf->chunk_len, num_q_heads, head_dim, pf->q_start);
}

extern "C" pa_status pa_paged_attention_mixed(const pa_decode_batch* dec,
                                              const pa_prefill_chunk* pf, pa_kv_view kv,
                                              int32_t num_q_heads, float scale, void* workspace,
                                              uint64_t workspace_bytes, uint32_t flags,
                                              void* stream) {
  return mixed_launch(dec, pf, kv, false, 1.0f, 1.0f, num_q_heads, scale, workspace,
                      workspace_bytes, flags, stream);
}

extern "C" pa_status pa_paged_attention_mixed_fp8(const pa_decode_batch* dec,
                                                  const pa_prefill_chunk* pf, pa_kv_view_fp8 kv,
                                                  int32_t num_q_heads, float scale,
                                                  void* workspace, uint64_t workspace_bytes,
                                                  uint32_t flags, void* stream) {
  const pa_kv_view v{reinterpret_cast<pa_half*>(kv.k_pool), reinterpret_cast<pa_half*>(kv.v_pool),
                     kv.num_blocks, kv.block_size, kv.num_kv_heads, kv.head_dim};
  return mixed_launch(dec, pf, v, true, kv.k_scale, kv.v_scale, num_q_heads, scale, workspace,
                      workspace_bytes, flags, stream);
}
