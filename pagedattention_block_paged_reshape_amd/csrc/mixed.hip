// Mixed decode + prefill launch on gfx950.
//
// Mixed step: the decode units of a batch and the tiles of one prefill chunk
// in one launch over one pool (a scheduler step runs both kinds of work in
// one forward pass: ta-paperlens "scheduler skeleton"; techfeed.io ngrok
// summary, "the scheduler").  Workgroups of the prefill launch's size (8
// wavefronts with fp16 pools, 4 with FP8 ones); the first pf_wgs take prefill
// tiles (kv head fastest, then query tile, then key split, as the prefill
// launch's grid), the rest decode units, one per wavefront pair (so 4 or 2
// per workgroup), each as in the grid form.  The prefill tiles, being the
// long work, start first; decode units fill the CUs as tiles retire, so the
// chunk's ragged end and the launch gap between the two kinds of work
// overlap with memory-bound decode.  Decode unit t of kv head g is entry t
// of the work list; the workgroup that holds entries P*j .. P*j + P - 1 of kv
// head g (P pairs) is number pf_wgs + j*n_kv + g, so with 8 kv heads and
// pf_wgs a multiple of 8 each head's decode units land on one XCD, as in the
// decode launch.
#include <type_traits>

#include "decode_core.h"
#include "prefill_tile.h"

namespace pa {

// Threads of a mixed workgroup: the prefill launch's workgroup size.
template <bool FP8>
constexpr int mixed_threads() {
  return FP8 ? kPfThreads : kPfPPThreads;
}

// LDS of a mixed workgroup: one prefill tile's, or P decode units' merge
// states ([pair][wave][16] max and sum, [pair][wave][G <= 16][D + 4] O^T rows).
template <int D, int P>
struct MixedDecodeLds {
  __attribute__((aligned(16))) float o[P][kDecodeWaves * 16 * (D + 4)];
  float m[P][kDecodeWaves * 16];
  float l[P][kDecodeWaves * 16];
  int arrive[P];
  int bad[P];
};

template <int D, bool FP8>
union MixedLds {
  static constexpr int P = mixed_threads<FP8>() / (kDecodeWaves * kWave);  // decode units
  typename std::conditional<FP8, PrefillLds<D>, PrefillLdsPP<D>>::type pf;
  MixedDecodeLds<D, P> dec;
};

template <int D, bool KEEP, bool FP8>
__global__ __launch_bounds__(mixed_threads<FP8>()) void mixed_step_kernel(
    PrefillArgs pa, int32_t pf_wgs, int32_t pf_qtiles, DecodeArgs da,
    const int32_t* __restrict__ items, int32_t n_items) {
  __shared__ MixedLds<D, FP8> lds;
  constexpr int P = MixedLds<D, FP8>::P;
  const int wg = blockIdx.x;
  if (wg < pf_wgs) {
    const int rest = wg / pa.n_kv;
    // FP8: no raised wave priority here, unlike the prefill launch: tiles
    // that share CUs with decode units starved them (measured on the
    // long-context step: 650 us with the prefill launch's priorities, also
    // when decode units ran at a higher priority, vs 607 us without).  The
    // fp16 tile fills its CU alone (two wavefronts per SIMD at ~211 VGPRs).
    if constexpr (FP8)
      prefill_tile<D, 0, FP8>(pa, wg % pa.n_kv, rest % pf_qtiles, rest / pf_qtiles, lds.pf);
    else
      prefill_tile_pp<D>(pa, wg % pa.n_kv, rest % pf_qtiles, rest / pf_qtiles, lds.pf);
    return;
  }
  if (threadIdx.x < P) {
    lds.dec.arrive[threadIdx.x] = 0;
    lds.dec.bad[threadIdx.x] = 0;
  }
  __syncthreads();
  const int j = wg - pf_wgs;
  const int pair = uniform(threadIdx.x >> 7);
  const int wave = uniform((threadIdx.x >> 6) & 1);
  const int lane = threadIdx.x & 63;
  const int g = j % da.n_kv;
  const int t = P * (j / da.n_kv) + pair;
  if (t >= n_items) return;
  const Unit u = make_entry_unit(da, static_cast<uint32_t>(scalar_load(items, t)), wave, lane);
  const Unit nx = no_unit();
  typedef TileRegs<D, FP8> TR;
  f16x8 qf[D / 32];
  typename TR::K kA[TR::NB * TR::NK], kB[TR::NB * TR::NK];
  typename TR::V vA[TR::NB * TR::NV], vB[TR::NB * TR::NV];
  if (u.cnt > 0) {
    load_q<D>(da, g, u.b, lane, qf);
    load_set<D, KEEP, FP8>(da, g, u, nx, 0, true, lane, kA, vA);
  }
  WaveState<D> st;
  run_unit<D, KEEP, FP8>(da, g, wave, lane, u, nx, qf, kA, vA, kB, vB, st);
  const MergeSlot<D> ms{lds.dec.m[pair], lds.dec.l[pair], lds.dec.o[pair], &lds.dec.arrive[pair],
                        &lds.dec.bad[pair]};
  if (post_state<D>(ms, st, da.G, wave, lane, u.bad) && u.ok)
    merge_store<D, FP8>(da, ms, g, u.b, u.p, u.L, u.n_parts, lane);
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

template <bool KEEP, bool FP8>
static void launch_step(int D, dim3 grid, hipStream_t s, const PrefillArgs& pa, int32_t pf_wgs,
                        int32_t qtiles, const DecodeArgs& da, const int32_t* items,
                        int32_t n_items) {
  const dim3 block(mixed_threads<FP8>());
  if (D == 128)
    mixed_step_kernel<128, KEEP, FP8><<<grid, block, 0, s>>>(pa, pf_wgs, qtiles, da, items,
                                                             n_items);
  else
    mixed_step_kernel<64, KEEP, FP8><<<grid, block, 0, s>>>(pa, pf_wgs, qtiles, da, items,
                                                            n_items);
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
  // decode units per workgroup: one per wavefront pair
  const int P = (fp8 ? mixed_threads<true>() : mixed_threads<false>()) / (kDecodeWaves * kWave);
  const int64_t dec_wgs =
      dec->batch > 0 ? static_cast<int64_t>(kv.num_kv_heads) * ((dec->n_items + P - 1) / P) : 0;
  if (pf_wgs + dec_wgs > 0x7FFFFFFF) return PA_ERR_INVALID;
  if (pf_wgs + dec_wgs == 0) return PA_OK;
  const bool keep = (flags & PA_DECODE_KEEP_KV) != 0;
  const int D = kv.head_dim;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<uint32_t>(pf_wgs + dec_wgs));
  const int32_t qtiles = static_cast<int32_t>(pgrid.y);
  const int32_t n_items = dec->batch > 0 ? dec->n_items : 0;
  const int32_t pw = static_cast<int32_t>(pf_wgs);
  if (fp8) {
    if (keep)
      launch_step<true, true>(D, grid, s, pa, pw, qtiles, da, dec->work_items, n_items);
    else
      launch_step<false, true>(D, grid, s, pa, pw, qtiles, da, dec->work_items, n_items);
  } else {
    if (keep)
      launch_step<true, false>(D, grid, s, pa, pw, qtiles, da, dec->work_items, n_items);
    else
      launch_step<false, false>(D, grid, s, pa, pw, qtiles, da, dec->work_items, n_items);
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
