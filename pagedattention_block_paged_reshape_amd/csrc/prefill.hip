// Causal chunked-prefill attention over the paged cache on gfx950.
//
// What is computed (techfeed.io ngrok summary, scheduler section: a very long
// prompt, e.g. 50,000 tokens, is split into chunks that fit the token budget
// and processed over several forward passes; ta-paperlens, "prefill grows
// with the square of the prompt length", FIG 1): a chunk of C query rows at
// absolute positions q_start + r attends, causally, to keys 0..q_start + r of
// its request, every key read through the request's block table (the
// chunk's own K/V were stored first).  Unlike decode, each K/V tile is
// reused by many query rows, so this is a dense QK^T / PV contraction and runs
// on the matrix cores (ta-paperlens, "prefill and decode": prefill is
// compute-bound).
//
// Design (MI355X):
//  * "M-rows" = query rows x the G query heads of one kv head; a wavefront
//    owns 32 M-rows as two 16-wide MFMA tiles.  Grid = (kv head, query tile,
//    key split); blockIdx.x = kv head puts each head on one XCD so that every
//    query tile and split of that head shares one L2 for the same K/V blocks.
//  * Keys advance 64 at a time (4 blocks).  fp16 pools (prefill_tile_pp): 8
//    wavefronts over 256 M-rows, in two groups that alternate between matrix
//    products and softmax at every phase (ping-pong), so that each SIMD's
//    matrix core is fed by one group while the other computes its
//    exponentials; the 4 K and 4 V tiles of a step are copied from HBM
//    straight into LDS (global -> LDS loads) in the pool's tile order, two
//    phases ahead of their first reader.  FP8 pools (prefill_tile): 4
//    wavefronts over 128 M-rows; the tiles are gathered into registers one
//    step ahead, converted, and stored to LDS in logical order (K as [key][D],
//    V^T as [D][key] in the score accumulators' key order, rows padded so the
//    MFMA operand reads are bank-conflict free).
//  * S^T = K . Q^T (keys x M-rows, 16x16x32 f16 MFMA); online softmax in fp32
//    base 2 per M-row; P^T goes straight from the score accumulators into the
//    B operand of O^T += V^T . P^T.  Only the steps that cross the causal
//    diagonal evaluate the mask.
//  * The key range is split over gridDim.z workgroups so that the grid has
//    several hundred workgroups; partial (o, m, l) are merged by log-sum-exp
//    in a second kernel, as in decode.
#include "prefill_tile.h"

namespace pa {

// Wave priority of the tile's phases (prefill_tile's PRIO bits): raised
// during the softmax and the PV products.  Two tile workgroups share each
// SIMD; letting the wavefront that is past its score products issue first
// keeps the matrix pipe fed while the other one computes its scores.
// Measured on the long-context chunk: 474 us vs 498 us with no priority
// (PV alone 481-483 us, scores alone 510 us, scores + PV 502 us).
constexpr int kPfPrio = kPfPrioSoftmax | kPfPrioPV;

template <int D, bool FP8>
__global__ __launch_bounds__(256) void prefill_chunk_kernel(PrefillArgs a) {
  __shared__ PrefillLds<D> lds;
  prefill_tile<D, kPfPrio, FP8>(a, blockIdx.x, blockIdx.y, blockIdx.z, lds);
}

// fp16 pools: the ping-pong tile, one 8-wavefront workgroup per 256 M-rows.
template <int D>
__global__ __launch_bounds__(kPfPPThreads) void prefill_chunk_pp_kernel(PrefillArgs a) {
  __shared__ PrefillLdsPP<D> lds;
  prefill_tile_pp<D>(a, blockIdx.x, blockIdx.y, blockIdx.z, lds);
}

// Merge the key splits of each (row, head) by log-sum-exp.
template <int D>
__global__ __launch_bounds__(64) void prefill_reduce_kernel(int32_t chunk_len, int32_t n_q,
                                                            int32_t splits,
                                                            const float* __restrict__ ws_o,
                                                            const float* __restrict__ ws_m,
                                                            const float* __restrict__ ws_l,
                                                            f16* __restrict__ out) {
  prefill_reduce_row<D>(chunk_len, n_q, splits, ws_o, ws_m, ws_l, out, blockIdx.x, blockIdx.y);
}

// Both pool types: checks, then the chunk kernel and (with key splits) the
// merge.  k_pool / v_pool hold fp16 values or (fp8) E4M3 codes.
static pa_status prefill_launch(pa_half* out, const pa_half* q, const pa_kv_view& kv, bool fp8,
                                float k_scale, float v_scale, const int32_t* table,
                                int32_t table_len, int32_t q_start, int32_t chunk_len,
                                int32_t num_q_heads, float scale, void* workspace,
                                uint64_t workspace_bytes, void* stream) {
  if (fp8 && !(k_scale > 0.0f && k_scale <= 3.0e38f && v_scale > 0.0f && v_scale <= 3.0e38f))
    return PA_ERR_INVALID;
  PrefillArgs a{};
  dim3 grid;
  const pa_status st = prefill_prepare(out, q, kv, table, table_len, q_start, chunk_len,
                                       num_q_heads, scale, workspace, workspace_bytes, a, grid);
  if (st != PA_OK || chunk_len == 0) return st;
  a.v_scale = 1.0f;
  if (fp8) {
    a.kp8 = reinterpret_cast<const uint8_t*>(kv.k_pool);
    a.vp8 = reinterpret_cast<const uint8_t*>(kv.v_pool);
    a.kp = a.vp = nullptr;
    // a score is scale * q . (code * k_scale): k_scale joins the exponent's factor
    a.scale_log2 *= k_scale;
    a.v_scale = v_scale;
  }
  const int D = kv.head_dim;
  const int splits = a.splits;
  float* ws_o = a.ws_o;
  float* ws_m = a.ws_m;
  float* ws_l = a.ws_l;
  f16* oo = a.out;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the fp16 tile covers 256 M-rows: half as many query tiles
  dim3 grid_pp = grid;
  grid_pp.y = static_cast<uint32_t>((chunk_len + kPfPPMRows / a.G - 1) / (kPfPPMRows / a.G));
  if (D == 128) {
    if (fp8)
      prefill_chunk_kernel<128, true><<<grid, dim3(kPfThreads), 0, s>>>(a);
    else
      prefill_chunk_pp_kernel<128><<<grid_pp, dim3(kPfPPThreads), 0, s>>>(a);
  } else {
    if (fp8)
      prefill_chunk_kernel<64, true><<<grid, dim3(kPfThreads), 0, s>>>(a);
    else
      prefill_chunk_pp_kernel<64><<<grid_pp, dim3(kPfPPThreads), 0, s>>>(a);
  }
  if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  if (splits > 1) {
    const dim3 rgrid(static_cast<uint32_t>(num_q_heads), static_cast<uint32_t>(chunk_len));
    if (D == 128)
      prefill_reduce_kernel<128><<<rgrid, dim3(64), 0, s>>>(chunk_len, num_q_heads, splits,
                                                            ws_o, ws_m, ws_l, oo);
    else
      prefill_reduce_kernel<64><<<rgrid, dim3(64), 0, s>>>(chunk_len, num_q_heads, splits,
                                                           ws_o, ws_m, ws_l, oo);
  }
  return launch_status();
}

}  // namespace pa

using namespace pa;

extern "C" uint64_t pa_prefill_workspace_bytes(int32_t chunk_len, int32_t num_q_heads,
                                               int32_t head_dim, int32_t q_start) {
  return prefill_ws_bytes(chunk_len, num_q_heads, head_dim, q_start);
}

extern "C" pa_status pa_paged_attention_prefill(pa_half* out, const pa_half* q, pa_kv_view kv,
                                                const int32_t* table, int32_t table_len,
                                                int32_t q_start, int32_t chunk_len,
                                                int32_t num_q_heads, float scale,
                                                void* workspace, uint64_t workspace_bytes,
                                                void* stream) {
  return prefill_launch(out, q, kv, false, 1.0f, 1.0f, table, table_len, q_start, chunk_len,
                        num_q_heads, scale, workspace, workspace_bytes, stream);
}

extern "C" pa_status pa_paged_attention_prefill_fp8(pa_half* out, const pa_half* q,
                                                    pa_kv_view_fp8 kv, const int32_t* table,
                                                    int32_t table_len, int32_t q_start,
                                                    int32_t chunk_len, int32_t num_q_heads,
                                                    float scale, void* workspace,
                                                    uint64_t workspace_bytes, void* stream) {
  const pa_kv_view v{reinterpret_cast<pa_half*>(kv.k_pool), reinterpret_cast<pa_half*>(kv.v_pool),
                     kv.num_blocks, kv.block_size, kv.num_kv_heads, kv.head_dim};
  return prefill_launch(out, q, v, true, kv.k_scale, kv.v_scale, table, table_len, q_start,
                        chunk_len, num_q_heads, scale, workspace, workspace_bytes, stream);
}
