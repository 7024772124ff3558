// Paged decode attention on gfx950: one step of attention for every running
// request, reading K and V through the request's block table.
//
// What is computed (ta-paperlens "LLM serving from scratch", "fragmentation
// and PagedAttention": the attention kernel follows the logical-to-physical
// table and gathers K and V while it computes; media.tcdigital.jp, "logical
// and physical block mapping"): for request i, query head h, kv head
// g = h / G,
//     out[i][h] = sum_j softmax_j(scale * q[i][h] . K_j) * V_j,  j < len_i,
// token j living in physical block table[i][j/16], slot j%16.  Decode reads
// the whole cache once per step and does little arithmetic per byte
// (ta-paperlens, "prefill and decode"), so this kernel is built to stream the
// pool at HBM rate.
//
// Design (MI355X):
//  * One workgroup (4 wavefronts) per (kv head, request, partition of
//    `part_blocks` blocks).  blockIdx.x is the kv head, so with 8 kv heads
//    each head's workgroups land on one XCD (workgroups are dealt to the 8
//    XCDs round-robin), keeping any shared-prefix blocks of that head in one
//    L2.
//  * The G query heads that share a kv head are the 16 columns of a
//    16x16 MFMA tile (padded when G < 16), so each K/V byte is read once per
//    kv head, not once per query head.
//  * Each wavefront takes every 4th block of the partition.  A block's K tile
//    ([16 tokens][D], 16*D*2 bytes contiguous) is loaded straight into the
//    MFMA A-operand registers (16 B per lane per K-step): S^T = K . Q^T gives
//    lane l the scores of 4 tokens for query head l%16.  Those scores, after
//    the online-softmax update, are already laid out as the B operand of
//    O^T += V^T . P^T, whose A operand is the V tile ([D][16 tokens]
//    contiguous, 8 B per lane per MFMA).  No LDS round trip is needed in the
//    main loop; the next block's tiles are in flight while the current one
//    is computed.
//  * Softmax runs in fp32 in base 2 (scores pre-multiplied by scale*log2 e);
//    the per-head running max is reduced across the 4 lane groups with two
//    xor shuffles, the running sum is kept per lane and reduced at the end.
//  * The 4 wavefronts' states are merged through LDS.  A request that fits in
//    one partition writes its fp16 output directly; longer ones write an fp32
//    partial (o normalised, m, l) that the reduce kernel merges by
//    log-sum-exp.
#include <math.h>

#include "pa_device.h"

namespace pa {

constexpr int kDecodeWaves = 4;

template <int D>
__global__ __launch_bounds__(256) void decode_partition_kernel(
    const f16* __restrict__ q, const f16* __restrict__ kp, const f16* __restrict__ vp,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ seq_lens,
    int32_t max_blocks, int32_t num_blocks, int32_t n_kv, int32_t G, float scale_log2,
    int32_t part_blocks, int32_t p_max, f16* __restrict__ out, float* __restrict__ ws_o,
    float* __restrict__ ws_m, float* __restrict__ ws_l) {
  constexpr int KS = D / 32;  // K-steps of the score MFMA
  constexpr int DT = D / 16;  // 16-wide dimension tiles of the output
  const int g = blockIdx.x;
  const int b = blockIdx.y;
  const int p = blockIdx.z;
  const int n_q = n_kv * G;

  int L = seq_lens[b];
  bool bad = false;
  if (L < 0) {
    L = 0;
    bad = true;
  }
  if (L > max_blocks * kBlock) {
    L = max_blocks * kBlock;
    bad = true;
  }
  const int part_tokens = part_blocks * kBlock;
  if (L > p_max * part_tokens) {  // longer than the max_seq_len the grid was sized for
    L = p_max * part_tokens;
    bad = true;
  }
  const int n_parts = (L + part_tokens - 1) / part_tokens;

  if (L == 0) {
    if (p == 0) {
      const float fill = bad ? __builtin_nanf("") : 0.0f;
      for (int i = threadIdx.x; i < G * D; i += blockDim.x)
        out[(static_cast<int64_t>(b) * n_q + g * G + i / D) * D + (i % D)] = static_cast<f16>(fill);
    }
    return;
  }
  if (p >= n_parts) return;

  const int wave = uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;  // token row of K loads; query head of Q / outputs
  const int lg = lane >> 4;   // lane group: which 8 (K) or 4 (V, P) k-values

  const int kb0 = p * part_blocks;
  const int kb_end = min(kb0 + part_blocks, (L + kBlock - 1) / kBlock);
  const int nb = kb_end - kb0;
  const int cnt = nb > wave ? (nb - wave + kDecodeWaves - 1) / kDecodeWaves : 0;

  // Q^T as the B operand: lane holds query head `col`, dims kk*32 + lg*8 .. +8.
  f16x8 qf[KS];
  {
    const f16* qrow = q + (static_cast<int64_t>(b) * n_q + g * G + col) * D + lg * 8;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      if (col < G)
        qf[kk] = *reinterpret_cast<const f16x8*>(qrow + kk * 32);
      else
        qf[kk] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }

  float m_run = -INFINITY;
  float l_run = 0.0f;
  f32x4 o[DT];
#pragma unroll
  for (int c = 0; c < DT; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int32_t* trow = tables + static_cast<int64_t>(b) * max_blocks;
  const int64_t head_tile = static_cast<int64_t>(n_kv);

  f16x8 kf[KS];
  f16x4 vf[DT];

  auto load_block = [&](int kb, f16x8* kd, f16x4* vd) {
    int pb = trow[kb];
    if (static_cast<uint32_t>(pb) >= static_cast<uint32_t>(num_blocks)) {
      bad = true;
      pb = 0;
    }
    const int64_t tile = static_cast<int64_t>(pb) * head_tile + g;
    const f16* kt = kp + tile * (kBlock * D) + col * D + lg * 8;
    const f16* vt = vp + tile * (kBlock * D) + col * kBlock + lg * 4;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) kd[kk] = *reinterpret_cast<const f16x8*>(kt + kk * 32);
#pragma unroll
    for (int c = 0; c < DT; ++c)
      vd[c] = *reinterpret_cast<const f16x4*>(vt + c * 16 * kBlock);
  };

  if (cnt > 0) load_block(kb0 + wave, kf, vf);

  for (int i = 0; i < cnt; ++i) {
    const int kb = kb0 + wave + kDecodeWaves * i;
    f16x8 kn[KS];
    f16x4 vn[DT];
    const bool more = i + 1 < cnt;
    if (more) load_block(kb + kDecodeWaves, kn, vn);

    // S^T tile: lane gets tokens kb*16 + 4*lg + j for query head col.
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) s = mfma16x16x32(kf[kk], qf[kk], s);

    const int tok0 = kb * kBlock + 4 * lg;
    const bool partial = (kb + 1) * kBlock > L;  // uniform: only the request's last block
    float sv[4];
    float mloc = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x = s[j] * scale_log2;
      sv[j] = (!partial || tok0 + j < L) ? x : -INFINITY;
      mloc = fmaxf(mloc, sv[j]);
    }
    mloc = wave_max_xor16_32(mloc);
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = exp2f(m_run - m_new);
    f16x4 pf;
    float psum = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f16 ph = static_cast<f16>(exp2f(sv[j] - m_new));
      pf[j] = ph;
      psum += static_cast<float>(ph);
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (partial) {
      // slots past the request's end hold stale bytes: zero them so that
      // 0 * (stale) cannot inject NaN/Inf
#pragma unroll
      for (int c = 0; c < DT; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (tok0 + j >= L) vf[c][j] = static_cast<f16>(0.0f);
    }
#pragma unroll
    for (int c = 0; c < DT; ++c) {
      o[c] *= alpha;
      o[c] = mfma16x16x16(vf[c], pf, o[c]);
    }
    if (more) {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) kf[kk] = kn[kk];
#pragma unroll
      for (int c = 0; c < DT; ++c) vf[c] = vn[c];
    }
  }

  l_run = wave_sum_xor16_32(l_run);

  // Merge the 4 wavefronts.  o[c][j] is O^T[c*16 + 4*lg + j][col].
  __shared__ float sm_m[kDecodeWaves][16];
  __shared__ float sm_l[kDecodeWaves][16];
  __shared__ float sm_o[kDecodeWaves][D][17];
  __shared__ int sm_bad;
  if (threadIdx.x == 0) sm_bad = 0;
  __syncthreads();
  if (lg == 0) {
    sm_m[wave][col] = m_run;
    sm_l[wave][col] = l_run;
  }
#pragma unroll
  for (int c = 0; c < DT; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) sm_o[wave][c * 16 + 4 * lg + j][col] = o[c][j];
  if (bad && lane == 0) sm_bad = 1;
  __syncthreads();
  const bool any_bad = sm_bad != 0;

  for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
    const int h = idx / D;
    const int dim = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) M = fmaxf(M, sm_m[w][h]);
    float wsum = 0.0f, acc = 0.0f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      const float e = exp2f(sm_m[w][h] - M);
      wsum += e * sm_l[w][h];
      acc += e * sm_o[w][dim][h];
    }
    float r = acc / wsum;
    if (any_bad) r = __builtin_nanf("");
    const int64_t qh = static_cast<int64_t>(b) * n_q + g * G + h;
    if (n_parts == 1) {
      out[qh * D + dim] = static_cast<f16>(r);
    } else {
      const int64_t slot = qh * p_max + p;
      ws_o[slot * D + dim] = r;
      if (dim == 0) {
        ws_m[slot] = any_bad ? __builtin_nanf("") : M;
        ws_l[slot] = wsum;
      }
    }
  }
}

// Merge the partitions of each (request, query head): with M = max_p m_p and
// w_p = l_p * 2^(m_p - M), out = sum_p w_p o_p / sum_p w_p.
template <int D>
__global__ __launch_bounds__(64) void decode_reduce_kernel(
    const int32_t* __restrict__ seq_lens, int32_t max_blocks, int32_t n_q, int32_t part_tokens,
    int32_t p_max, const float* __restrict__ ws_o, const float* __restrict__ ws_m,
    const float* __restrict__ ws_l, f16* __restrict__ out) {
  constexpr int PER = D / 64;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  int L = seq_lens[b];
  if (L < 0) return;                                    // partition kernel wrote NaN
  if (L > max_blocks * kBlock) L = max_blocks * kBlock;  // partials are NaN-flagged
  const int n_parts = min((L + part_tokens - 1) / part_tokens, p_max);
  if (n_parts <= 1) return;
  const int64_t base = (static_cast<int64_t>(b) * n_q + h) * p_max;
  float M = -INFINITY;
  for (int pp = 0; pp < n_parts; ++pp) M = fmaxf(M, ws_m[base + pp]);
  float wsum = 0.0f;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.0f;
  for (int pp = 0; pp < n_parts; ++pp) {
    const float w = ws_l[base + pp] * exp2f(ws_m[base + pp] - M);
    wsum += w;
    const float* op = ws_o + (base + pp) * D;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] += w * op[threadIdx.x + 64 * e];
  }
  const float inv = 1.0f / wsum;
  f16* orow = out + (static_cast<int64_t>(b) * n_q + h) * D;
#pragma unroll
  for (int e = 0; e < PER; ++e) orow[threadIdx.x + 64 * e] = static_cast<f16>(acc[e] * inv);
}

}  // namespace pa

using namespace pa;

extern "C" uint64_t pa_decode_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                              int32_t head_dim, int32_t max_seq_len,
                                              int32_t partition_size) {
  if (batch <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_seq_len <= 0 || partition_size <= 0)
    return 0;
  const uint64_t parts = (static_cast<uint64_t>(max_seq_len) + partition_size - 1) / partition_size;
  return static_cast<uint64_t>(batch) * num_q_heads * parts * (head_dim + 2) * sizeof(float);
}

extern "C" pa_status pa_paged_attention_decode(pa_half* out, const pa_half* q, pa_kv_view kv,
                                               const int32_t* tables, int32_t max_blocks,
                                               const int32_t* seq_lens, int32_t batch,
                                               int32_t num_q_heads, float scale,
                                               int32_t partition_size, int32_t max_seq_len,
                                               void* workspace, uint64_t workspace_bytes,
                                               void* stream) {
  if (kv.k_pool == nullptr || kv.v_pool == nullptr || kv.block_size != kBlock ||
      kv.num_blocks <= 0 || kv.num_kv_heads <= 0 || kv.num_kv_heads > 65535)
    return PA_ERR_INVALID;
  if (kv.head_dim != 64 && kv.head_dim != 128) return PA_ERR_INVALID;
  if (batch < 0 || batch > 65535 || max_blocks < 0 || max_seq_len < 0) return PA_ERR_INVALID;
  if (num_q_heads <= 0 || num_q_heads % kv.num_kv_heads != 0) return PA_ERR_INVALID;
  const int G = num_q_heads / kv.num_kv_heads;
  if (G > 16) return PA_ERR_INVALID;
  if (partition_size <= 0 || partition_size % kBlock != 0) return PA_ERR_INVALID;
  if (!(scale == scale)) return PA_ERR_INVALID;
  if (batch == 0) return PA_OK;
  if (out == nullptr || q == nullptr || tables == nullptr || seq_lens == nullptr ||
      !aligned16(q) || !aligned16(kv.k_pool) || !aligned16(kv.v_pool))
    return PA_ERR_INVALID;
  if (static_cast<int64_t>(max_seq_len) > static_cast<int64_t>(max_blocks) * kBlock)
    return PA_ERR_INVALID;
  const int part_blocks = partition_size / kBlock;
  const int p_max = max_seq_len == 0 ? 1 : (max_seq_len + partition_size - 1) / partition_size;
  if (p_max > 65535) return PA_ERR_INVALID;
  const int D = kv.head_dim;
  float *ws_o = nullptr, *ws_m = nullptr, *ws_l = nullptr;
  if (p_max > 1) {
    const uint64_t need =
        pa_decode_workspace_bytes(batch, num_q_heads, D, max_seq_len, partition_size);
    if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace))
      return PA_ERR_INVALID;
    const int64_t slots = static_cast<int64_t>(batch) * num_q_heads * p_max;
    ws_o = static_cast<float*>(workspace);
    ws_m = ws_o + slots * D;
    ws_l = ws_m + slots;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float scale_log2 = scale * 1.4426950408889634f;
  const dim3 grid(static_cast<uint32_t>(kv.num_kv_heads), static_cast<uint32_t>(batch),
                  static_cast<uint32_t>(p_max));
  const f16* qq = reinterpret_cast<const f16*>(q);
  const f16* kp = reinterpret_cast<const f16*>(kv.k_pool);
  const f16* vp = reinterpret_cast<const f16*>(kv.v_pool);
  f16* oo = reinterpret_cast<f16*>(out);
  if (D == 128)
    decode_partition_kernel<128><<<grid, dim3(256), 0, s>>>(
        qq, kp, vp, tables, seq_lens, max_blocks, kv.num_blocks, kv.num_kv_heads, G, scale_log2,
        part_blocks, p_max, oo, ws_o, ws_m, ws_l);
  else
    decode_partition_kernel<64><<<grid, dim3(256), 0, s>>>(
        qq, kp, vp, tables, seq_lens, max_blocks, kv.num_blocks, kv.num_kv_heads, G, scale_log2,
        part_blocks, p_max, oo, ws_o, ws_m, ws_l);
  if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  if (p_max > 1) {
    const dim3 rgrid(static_cast<uint32_t>(num_q_heads), static_cast<uint32_t>(batch));
    if (D == 128)
      decode_reduce_kernel<128><<<rgrid, dim3(64), 0, s>>>(
          seq_lens, max_blocks, num_q_heads, partition_size, p_max, ws_o, ws_m, ws_l, oo);
    else
      decode_reduce_kernel<64><<<rgrid, dim3(64), 0, s>>>(
          seq_lens, max_blocks, num_q_heads, partition_size, p_max, ws_o, ws_m, ws_l, oo);
  }
  return launch_status();
}
