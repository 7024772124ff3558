// Causal chunked-prefill attention tile over the paged cache (gfx950): the
// device code shared by the prefill launch and the mixed decode + prefill
// launch.  What is computed and how is described where the kernels are
// defined, in prefill.hip.
#pragma once

#include <math.h>

#include "pa_device.h"

namespace pa {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kPfThreads = 256;
// Phases of a key step whose wave priority prefill_tile raises (PRIO bits).
constexpr int kPfPrioScores = 1;   // S^T = K . Q^T products
constexpr int kPfPrioPV = 2;       // O^T += V^T . P^T products
constexpr int kPfPrioSoftmax = 4;  // online softmax between them
constexpr int kPfPrioStage = 8;    // barriers, LDS stores and next loads
constexpr int kPfMRows = 128;   // M-rows per workgroup
constexpr int kPfKeys = 64;     // keys per step
constexpr float kPfSumLimit = 32768.0f;  // bound on a lane's P sum of a row and step
constexpr int kPfMaxSplits = 32;
#ifndef PA_PF_TARGET_WGS
#define PA_PF_TARGET_WGS 512
#endif
constexpr int kPfTargetWgs = PA_PF_TARGET_WGS;

// Splits of the key range: enough workgroups to cover the 256 CUs twice.
__host__ __device__ inline int prefill_splits(int chunk_len, int n_q, int q_start) {
  const long long base = (static_cast<long long>(chunk_len) * n_q + kPfMRows - 1) / kPfMRows;
  long long s = (kPfTargetWgs + base - 1) / (base > 0 ? base : 1);
  const long long steps = (static_cast<long long>(q_start) + chunk_len + kPfKeys - 1) / kPfKeys;
  if (s > steps) s = steps;
  if (s > kPfMaxSplits) s = kPfMaxSplits;
  if (s < 1) s = 1;
  return static_cast<int>(s);
}

// LDS of one tile: the step's K rows and V^T rows, and the bad-entry flag.
template <int D>
struct PrefillLds {
  __attribute__((aligned(16))) f16 sk[kPfKeys * (D + 8)];
  __attribute__((aligned(16))) f16 sv[D * (kPfKeys + 8)];
  int bad;
};

// Arguments of one chunk: queries, pools, the request's table, geometry, and
// the output or (several key splits) the fp32 partials.
struct PrefillArgs {
  const f16* q;
  const f16* kp;
  const f16* vp;
  const int32_t* table;
  int32_t table_len;
  int32_t num_blocks;
  int32_t n_kv;
  int32_t G;
  int32_t q_start;
  int32_t chunk_len;
  float scale_log2;
  int32_t splits;
  f16* out;
  float* ws_o;
  float* ws_m;
  float* ws_l;
  // FP8 pools (E4M3 codes, one scale per pool): k_scale is folded into
  // scale_log2 by the host, v_scale multiplies the normalised output
  const uint8_t* kp8;
  const uint8_t* vp8;
  float v_scale;
};

// Four E4M3 codes (byte j of w is element j) as fp16 (exact: every E4M3
// value is an fp16 value).
__device__ __forceinline__ f16x4 pf_e4m3x4_to_f16(uint32_t w) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 r = {
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true))};
  return __builtin_bit_cast(f16x4, r);
}

// One key step's online softmax for a wavefront's two 16-row score tiles, in
// fp32 and base 2, against a per-row reference m (the exponent's offset):
// P = 2^(s * scale_log2 - m) rounded to fp16, with l (the sum of the rounded
// P, the weights the PV products use) and O accumulated against the same m.
// No row maximum is taken per step: a lane's sum of its 16 rounded P of a row
// bounds each of them, so while every such sum of the row stays within
// kPfSumLimit no P can overflow fp16 and m stays.  Otherwise, or while the row
// has no reference yet, m moves up to the row's maximum, l and O are rescaled
// by 2^(m_old - m_new) and the P recomputed: a wave-uniform branch, rare after
// a row's first keys.  A row's m depends only on that row's scores (the other
// rows of the wavefront keep theirs, a rescale by exactly 1), so any tiling
// of the rows gives the same bits.  Any reference gives the same o / l, and
// split partials store theirs with l.
template <int DT>
__device__ __forceinline__ void pf_softmax(const f32x4 (&s)[4][2], float scale_log2, int col,
                                          float (&m_run)[2], float (&l_run)[2],
                                          f32x4 (&o)[DT][2], f16x8 (&pb8)[2][2]) {
  float psum[2];
  auto exponents = [&]() {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const float m_use = m_run[nt] == -INFINITY ? 0.0f : m_run[nt];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          pb8[mt >> 1][nt][(mt & 1) * 4 + j] =
              static_cast<f16>(__builtin_amdgcn_exp2f(fmaf(s[mt][nt][j], scale_log2, -m_use)));
      // the rounded P summed two per instruction, in fp32
      float acc = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int h = 0; h < 4; ++h)
          acc = __builtin_amdgcn_fdot2(f16x2{pb8[ks][nt][2 * h], pb8[ks][nt][2 * h + 1]},
                                       f16x2{static_cast<f16>(1.0f), static_cast<f16>(1.0f)},
                                       acc, false);
      psum[nt] = acc;
    }
  };
  exponents();
  const uint64_t over0 =
      __builtin_amdgcn_ballot_w64(!(psum[0] <= kPfSumLimit) || m_run[0] == -INFINITY);
  const uint64_t over1 =
      __builtin_amdgcn_ballot_w64(!(psum[1] <= kPfSumLimit) || m_run[1] == -INFINITY);
  if ((over0 | over1) != 0) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const uint64_t over = nt == 0 ? over0 : over1;
      // the row of lane col is held by lanes col, col + 16, col + 32, col + 48
      const uint32_t rows = static_cast<uint32_t>(over | (over >> 16) | (over >> 32) | (over >> 48));
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) mx = fmaxf(mx, s[mt][nt][j]);
      // in base-2 units (scale_log2 > 0, so max(s) * c = max(s * c))
      const float m_row = wave_max_xor16_32(mx) * scale_log2;
      const float m_new = ((rows >> col) & 1u) != 0 ? fmaxf(m_run[nt], m_row) : m_run[nt];
      // hardware 2^x: results below 2^-126 flush to 0, which softmax ignores
      const float alpha = m_new == m_run[nt] || m_new == -INFINITY
                              ? 1.0f
                              : __builtin_amdgcn_exp2f(m_run[nt] - m_new);
      l_run[nt] *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt][nt] *= alpha;
      m_run[nt] = m_new;
    }
    exponents();
  }
  l_run[0] += psum[0];
  l_run[1] += psum[1];
}

// One workgroup's tile: kv head g, query tile qt, key split z.  All 256
// threads of the workgroup take part (it has two workgroup barriers per key
// step).
// Wave priority at the switch from phase FROM to phase TO of a key step
// (kPfPrio* bits of PRIO: priority 1, else 0).  Only a change emits an
// s_setprio, which the compiler does not schedule across.  The loop's first
// phase is entered from PV's level (priority 0 before the loop).
template <int PRIO, int FROM, int TO>
__device__ __forceinline__ void phase_prio() {
  constexpr int from = (PRIO & FROM) ? 1 : 0;
  constexpr int to = (PRIO & TO) ? 1 : 0;
  if constexpr (from != to) __builtin_amdgcn_s_setprio(to);
}

// PRIO: the kPfPrio* phases run at wave priority 1 (else 0).
template <int D, int PRIO, bool FP8 = false>
__device__ __forceinline__ void prefill_tile(const PrefillArgs& a, int g, int qt, int z,
                                             PrefillLds<D>& lds) {
  const f16* __restrict__ q = a.q;
  const f16* __restrict__ kp = a.kp;
  const f16* __restrict__ vp = a.vp;
  const int32_t* __restrict__ table = a.table;
  const int32_t table_len = a.table_len, num_blocks = a.num_blocks, n_kv = a.n_kv, G = a.G;
  const int32_t q_start = a.q_start, chunk_len = a.chunk_len, splits = a.splits;
  const float scale_log2 = a.scale_log2;
  f16* __restrict__ out = a.out;
  float* __restrict__ ws_o = a.ws_o;
  float* __restrict__ ws_m = a.ws_m;
  float* __restrict__ ws_l = a.ws_l;
  constexpr int KS = D / 32;       // K-steps over head_dim
  constexpr int DT = D / 16;       // dim tiles of O^T
  constexpr int KROW = D + 8;      // padded K row (halves)
  constexpr int VROW = kPfKeys + 8;  // padded V^T row (halves)
  constexpr int KCH = kPfKeys * D / 8 / kPfThreads;  // 16-B chunks per thread per tile set
  f16* const sk = lds.sk;
  f16* const sv = lds.sv;
  int& sbad = lds.bad;
  const int n_q = n_kv * G;
  const int QR = kPfMRows / G;  // query rows per tile
  const int r0 = qt * QR;
  const int seq_end = q_start + chunk_len;

  const int wave = uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int lg = lane >> 4;

  // keys this tile needs: 0 .. q_start + (last row) inclusive
  const int last_row = min(r0 + QR, chunk_len) - 1;
  const int key_end = q_start + last_row + 1;
  const int n_steps = (key_end + kPfKeys - 1) / kPfKeys;
  // Key steps of split z: the chunk's whole key range cut into `splits` equal
  // parts (one cut for every query tile, whatever its size, so that a row's
  // partials and their merge do not depend on the tiling), clipped to this
  // tile's keys.  A step past a row's last key adds nothing to it.
  const long long n_all = (static_cast<long long>(seq_end) + kPfKeys - 1) / kPfKeys;
  const int st0 = static_cast<int>((n_all * z) / splits);
  const int st1 = min(static_cast<int>((n_all * (z + 1)) / splits), n_steps);

  // M-rows of this lane for the two n-tiles, and their query rows / heads
  int mrow_r[2], mrow_h[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int m = wave * 32 + nt * 16 + col;
    mrow_h[nt] = m / QR;
    mrow_r[nt] = r0 + (m % QR);
  }

  // Q^T fragments (B operand): M-row's query, dims kk*32 + lg*8 .. +8
  f16x8 qf[2][KS];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int r = min(mrow_r[nt], chunk_len - 1);
    const f16* qrow = q + (static_cast<int64_t>(r) * n_q + g * G + mrow_h[nt]) * D + lg * 8;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) qf[nt][kk] = *reinterpret_cast<const f16x8*>(qrow + kk * 32);
  }

  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};
  f32x4 o[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) o[dt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (threadIdx.x == 0) sbad = 0;
  bool bad = false;

  // Register staging of one step's 4 K tiles and 4 V tiles.
  f16x8 rk[KCH], rv[KCH];
  // FP8 pools: a tile is 16 * D bytes = D chunks of 16 codes; thread t holds
  // chunk (t + 256u) % D of block (t + 256u) / D (uniform over a wavefront)
  constexpr int KCH8 = (kPfKeys / kBlock) * D / kPfThreads;
  u32x4 rk8[KCH8 > 0 ? KCH8 : 1], rv8[KCH8 > 0 ? KCH8 : 1];
  // Physical ids of a step's 4 blocks, read (clamped into the table; entries
  // past the sequence are never used) a step before their fetch.
  constexpr int kStepBlocks = kPfKeys / kBlock;
  auto read_ids = [&](int step, int (&ids)[kStepBlocks]) {
#pragma unroll
    for (int i = 0; i < kStepBlocks; ++i)
      ids[i] = scalar_load(table, min(step * kStepBlocks + i, table_len - 1));
  };
  // Chunk u of every thread lies in one block of the step, the same for the
  // whole wavefront (a block is kBlock * D / 8 >= 64 chunks), so the bounds
  // checks and the tail test are scalar.
  auto fetch = [&](int step, const int (&ids)[kStepBlocks]) {
    const int key0 = step * kPfKeys;
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int ci = threadIdx.x + kPfThreads * u;         // 16-byte chunk of the 4-tile set
      const int bi = uniform(ci / (kBlock * D / 8));       // which of the 4 blocks
      const int within = ci % (kBlock * D / 8);
      const int lb = key0 / kBlock + bi;                   // logical block
      const f16x8 zero = {0, 0, 0, 0, 0, 0, 0, 0};
      if (lb * kBlock >= seq_end || lb >= table_len) {
        rk[u] = zero;
        rv[u] = zero;
        continue;
      }
      int pb = ids[bi];
      if (static_cast<uint32_t>(pb) >= static_cast<uint32_t>(num_blocks)) {
        bad = true;
        pb = 0;
      }
      const int64_t tile = (static_cast<int64_t>(pb) * n_kv + g) * (kBlock * D);
      rk[u] = *reinterpret_cast<const f16x8*>(kp + tile + within * 8);
      f16x8 vv = *reinterpret_cast<const f16x8*>(vp + tile + within * 8);
      if (lb * kBlock + kBlock > seq_end) {
        // the sequence's last block: V chunk `within` holds two dims' values
        // for slots 4q .. 4q+3 (tile order [D/32][4][16][2][4]); zero the
        // slots past the end
        const int q4 = ((within >> 4) & 3) * 4;
        const int valid = seq_end - (lb * kBlock + q4);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if ((e & 3) >= valid) vv[e] = static_cast<f16>(0.0f);
      }
      rv[u] = vv;
    }
  };
  auto fetch8 = [&](int step, const int (&ids)[kStepBlocks]) {
    const int key0 = step * kPfKeys;
#pragma unroll
    for (int u = 0; u < KCH8; ++u) {
      const int ci = threadIdx.x + kPfThreads * u;
      const int bi = uniform(ci / D);
      const int within = ci % D;
      const int lb = key0 / kBlock + bi;
      if (lb * kBlock >= seq_end || lb >= table_len) {
        rk8[u] = u32x4{0u, 0u, 0u, 0u};
        rv8[u] = u32x4{0u, 0u, 0u, 0u};
        continue;
      }
      int pb = ids[bi];
      if (static_cast<uint32_t>(pb) >= static_cast<uint32_t>(num_blocks)) {
        bad = true;
        pb = 0;
      }
      const int64_t tile = (static_cast<int64_t>(pb) * n_kv + g) * (kBlock * D);
      rk8[u] = *reinterpret_cast<const u32x4*>(a.kp8 + tile + within * 16);
      u32x4 vv = *reinterpret_cast<const u32x4*>(a.vp8 + tile + within * 16);
      if (lb * kBlock + kBlock > seq_end) {
        // the sequence's last block: V chunk `within` holds slots 4q .. 4q+3
        // (q = (within/16) % 4), slot 4q + j in byte j of each dword; zero
        // the codes past the end (code 0 is +0)
        const int valid = seq_end - (lb * kBlock + ((within >> 4) & 3) * 4);
        const uint32_t keep =
            valid >= 4 ? 0xFFFFFFFFu : (valid <= 0 ? 0u : (1u << (8 * valid)) - 1u);
        vv &= u32x4{keep, keep, keep, keep};
      }
      rv8[u] = vv;
    }
  };
  // FP8 chunk `within` of block bi: K slot within%16, dims 8*d8 .. +8 (bytes
  // 0-7) and 8*(d8+4) .. +8 (bytes 8-15), d8 = 8*(within/64) + (within/16)%4;
  // V dims c0 + 32*(t/2) + 16*(t%2) (dword t) at slots 4q .. 4q+3,
  // c0 = 64*(within/64) + within%16.  Widened to fp16 into the same LDS rows
  // as the fp16 path.
  auto stash8 = [&]() {
#pragma unroll
    for (int u = 0; u < KCH8; ++u) {
      const int ci = threadIdx.x + kPfThreads * u;
      const int bi = ci / D;
      const int within = ci % D;
      const int key = bi * kBlock + (within & 15);
      const int d8 = 8 * (within >> 6) + ((within >> 4) & 3);
      const u32x4 kw = rk8[u];
      const f16x4 k0 = pf_e4m3x4_to_f16(kw[0]), k1 = pf_e4m3x4_to_f16(kw[1]);
      const f16x4 k2 = pf_e4m3x4_to_f16(kw[2]), k3 = pf_e4m3x4_to_f16(kw[3]);
      *reinterpret_cast<f16x8*>(sk + key * KROW + d8 * 8) =
          f16x8{k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
      *reinterpret_cast<f16x8*>(sk + key * KROW + (d8 + 4) * 8) =
          f16x8{k2[0], k2[1], k2[2], k2[3], k3[0], k3[1], k3[2], k3[3]};
      const int c0 = 64 * (within >> 6) + (within & 15);
      const int q4 = (within >> 4) & 3;
      const int kpos = (bi >> 1) * 32 + q4 * 8 + (bi & 1) * 4;
      const u32x4 vw = rv8[u];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int dim = c0 + 32 * (t >> 1) + 16 * (t & 1);
        *reinterpret_cast<f16x4*>(sv + dim * VROW + kpos) = pf_e4m3x4_to_f16(vw[t]);
      }
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int ci = threadIdx.x + kPfThreads * u;
      const int bi = ci / (kBlock * D / 8);
      const int within = ci % (kBlock * D / 8);
      // K chunk `within` = dims (within/16)*8 .. +8 of slot within%16
      const int key = bi * kBlock + (within & 15);
      const int d8 = within >> 4;
      *reinterpret_cast<f16x8*>(sk + key * KROW + d8 * 8) = rk[u];
      // V chunk `within` = dims c2*32 + dd and c2*32 + 16 + dd, slots 4q .. +4.
      // V^T rows keep each 32-key half in the order the score accumulators
      // hold P^T: key 16h + 4q + j of the half sits at 8q + 4h + j, so one
      // 16-byte read gives a lane its 8 keys of the PV operand.
      const int dim = (within >> 6) * 32 + (within & 15);
      const int q4 = (within >> 4) & 3;
      const int kpos = (bi >> 1) * 32 + q4 * 8 + (bi & 1) * 4;
      const f16x8 vv = rv[u];
      *reinterpret_cast<f16x4*>(sv + dim * VROW + kpos) = f16x4{vv[0], vv[1], vv[2], vv[3]};
      *reinterpret_cast<f16x4*>(sv + (dim + 16) * VROW + kpos) = f16x4{vv[4], vv[5], vv[6], vv[7]};
    }
  };

  int ids[kStepBlocks];
  if (st0 < st1) {
    read_ids(st0, ids);
    if constexpr (FP8) fetch8(st0, ids); else fetch(st0, ids);
  }
  if (st0 + 1 < st1) read_ids(st0 + 1, ids);
  for (int step = st0; step < st1; ++step) {
    phase_prio<PRIO, kPfPrioPV, kPfPrioStage>();
    __syncthreads();  // previous step's LDS reads are done
    if constexpr (FP8) stash8(); else stash();
    __syncthreads();
    if (step + 1 < st1) {
      if constexpr (FP8) fetch8(step + 1, ids); else fetch(step + 1, ids);
    }

    const int key0 = step * kPfKeys;
    // scores S^T[key][M-row]: 4 key tiles x 2 M-row tiles
    phase_prio<PRIO, kPfPrioStage, kPfPrioScores>();
    f32x4 s[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f16x8 ka[KS];
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        ka[kk] = *reinterpret_cast<const f16x8*>(sk + (mt * 16 + col) * KROW + kk * 32 + lg * 8);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) acc = mfma16x16x32(ka[kk], qf[nt][kk], acc);
        s[mt][nt] = acc;
      }
    }

    phase_prio<PRIO, kPfPrioScores, kPfPrioSoftmax>();
    if (step + 2 < st1) read_ids(step + 2, ids);

    // causal mask, on the raw scores, only where the step crosses the
    // diagonal of this tile (a uniform branch: most steps skip it)
    if (key0 + kPfKeys - 1 > q_start + r0) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int limit = q_start + min(mrow_r[nt], chunk_len - 1);  // last key allowed
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (key0 + mt * 16 + 4 * lg + j > limit) s[mt][nt][j] = -INFINITY;
      }
    }
    f16x8 pb8[2][2];  // [k-step of PV][n-tile]
    pf_softmax<DT>(s, scale_log2, col, m_run, l_run, o, pb8);

    // O^T[dim][M-row] += V^T[dim][key] . P^T[key][M-row]
    phase_prio<PRIO, kPfPrioSoftmax, kPfPrioPV>();
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const f16x8 va =
            *reinterpret_cast<const f16x8*>(sv + (dt * 16 + col) * VROW + ks * 32 + 8 * lg);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) o[dt][nt] = mfma16x16x32(va, pb8[ks][nt], o[dt][nt]);
      }
    }
  }
  if constexpr ((PRIO & kPfPrioPV) != 0) __builtin_amdgcn_s_setprio(0);

  if (bad) sbad = 1;
  __syncthreads();
  const bool any_bad = sbad != 0;

#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const float l = wave_sum_xor16_32(l_run[nt]);
    const int r = mrow_r[nt];
    if (r >= chunk_len) continue;
    const int head = g * G + mrow_h[nt];
    const float inv = l > 0.0f ? (FP8 ? a.v_scale / l : 1.0f / l) : 0.0f;
    const int64_t qh = static_cast<int64_t>(r) * n_q + head;
    if (splits == 1) {
      f16* orow = out + qh * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        f16x4 h4;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          h4[j] = static_cast<f16>(any_bad ? __builtin_nanf("") : o[dt][nt][j] * inv);
        *reinterpret_cast<f16x4*>(orow + dt * 16 + 4 * lg) = h4;
      }
    } else {
      const int64_t slot = static_cast<int64_t>(z) * chunk_len * n_q + qh;
      float* orow = ws_o + slot * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(orow + dt * 16 + 4 * lg) =
          o[dt][nt] * inv;
      if (lg == 0) {
        ws_m[slot] = any_bad ? __builtin_nanf("") : m_run[nt];
        ws_l[slot] = l;
      }
    }
  }
}


// The fp16 tile of the prefill launch: 8 wavefronts over 256 M-rows (32 per
// wavefront, as in prefill_tile), in two groups of 4 that share each SIMD.
constexpr int kPfPPThreads = 512;
constexpr int kPfPPMRows = 256;

// LDS of one such tile: two buffers of a step's 4 K tiles and 4 V tiles, each
// in the pool's own tile order (so that they can be copied from HBM as they
// are), and the bad-entry flag.
template <int D>
struct PrefillLdsPP {
  __attribute__((aligned(16))) f16 kv[2][2][kPfKeys * D];  // [buffer][K, V][4 tiles]
  int bad;
};

// s_waitcnt immediate that waits for every outstanding vector memory access:
// vmcnt 0, with expcnt and lgkmcnt at their maxima (not waited on).
constexpr int kVmcnt0 = 0x0F70;

// One workgroup's fp16 tile (kv head g, query tile qt, key split z) with the
// two wavefront groups in ping-pong.  Phases are separated by workgroup
// barriers; in each phase one group runs matrix products (step j - 1's PV
// products, then step j's scores) while the other runs a step's softmax on
// the vector ALUs, and the roles swap at the next phase, so that the matrix
// cores of every SIMD are fed by one wavefront or the other.  Group 0 takes
// its product phase for step j at phase 2j, group 1 one phase later.
//
// K and V tiles are copied from HBM straight into LDS with gfx950's global ->
// LDS loads (16 bytes per lane, no staging registers), in the pool's tile
// order; the operand reads below are laid out for that order.  At every even
// phase 2j, group 1 requests K(j + 1) and V(j); both have landed before phase
// 2j + 2, the first that reads them, in the buffers that K(j - 1) and
// V(j - 2) left at phase 2j - 1.  A step that is not 4 whole blocks (the
// sequence's last one or two) goes through registers instead, so that V slots
// past the end (and blocks past it) are zeroed: 0 * stale bytes could inject
// NaN into the products.
//
// Per row the arithmetic is prefill_tile's, in the same order: the same
// products, pf_softmax, the same PV order; the results are the same bits.
template <int D>
__device__ __forceinline__ void prefill_tile_pp(const PrefillArgs& a, int g, int qt, int z,
                                                PrefillLdsPP<D>& lds) {
  const f16* __restrict__ q = a.q;
  const f16* __restrict__ kp = a.kp;
  const f16* __restrict__ vp = a.vp;
  const int32_t* __restrict__ table = a.table;
  const int32_t table_len = a.table_len, num_blocks = a.num_blocks, n_kv = a.n_kv, G = a.G;
  const int32_t q_start = a.q_start, chunk_len = a.chunk_len, splits = a.splits;
  const float scale_log2 = a.scale_log2;
  f16* __restrict__ out = a.out;
  constexpr int KS = D / 32;                       // K-steps over head_dim
  constexpr int DT = D / 16;                       // dim tiles of O^T
  constexpr int TILE = kBlock * D;                 // halves per (block, kv head) tile
  constexpr int CPT = TILE / 8;                    // 16-byte chunks per tile
  constexpr int KCH = kPfKeys * D / 8 / 256;       // chunks per copying thread per tile set
  constexpr int TPB = 256 / CPT;                   // tiles one round of 256 threads covers
  constexpr int kStepBlocks = kPfKeys / kBlock;
  int& sbad = lds.bad;
  const int n_q = n_kv * G;
  const int QR = kPfPPMRows / G;  // query rows per tile
  const int r0 = qt * QR;
  const int seq_end = q_start + chunk_len;
  const int wave = uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int lg = lane >> 4;
  const int last_row = min(r0 + QR, chunk_len) - 1;
  const int key_end = q_start + last_row + 1;
  const int n_steps = (key_end + kPfKeys - 1) / kPfKeys;
  // Key steps of split z: the chunk's whole key range cut into `splits` equal
  // parts (one cut for every query tile, whatever its size, so that a row's
  // partials and their merge do not depend on the tiling), clipped to this
  // tile's keys.  A step past a row's last key adds nothing to it.
  const long long n_all = (static_cast<long long>(seq_end) + kPfKeys - 1) / kPfKeys;
  const int st0 = static_cast<int>((n_all * z) / splits);
  const int st1 = min(static_cast<int>((n_all * (z + 1)) / splits), n_steps);

  int mrow_r[2], mrow_h[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int m = wave * 32 + nt * 16 + col;
    mrow_h[nt] = m / QR;
    mrow_r[nt] = r0 + (m % QR);
  }
  f16x8 qf[2][KS];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int r = min(mrow_r[nt], chunk_len - 1);
    const f16* qrow = q + (static_cast<int64_t>(r) * n_q + g * G + mrow_h[nt]) * D + lg * 8;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) qf[nt][kk] = *reinterpret_cast<const f16x8*>(qrow + kk * 32);
  }
  // the query fragments in before the loop, so that no wait inside it is on
  // their account
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};
  f32x4 o[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) o[dt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (threadIdx.x == 0) sbad = 0;
  bool bad = false;

  // Copies by group 1's 256 threads: chunk u of such a thread is chunk
  // `within` of block u * TPB + tsub of the step.
  const int ctid = static_cast<int>(threadIdx.x) & 255;
  const int tsub = TPB > 1 ? uniform(ctid / CPT) : 0;
  const int within = ctid % CPT;
  const int wchunk0 = uniform(within - lane);  // the wavefront's first chunk
  const uint32_t lane_byte = static_cast<uint32_t>(within) * 16u;
  const uint64_t head_off = static_cast<uint64_t>(g) * TILE;
  const uint32_t block_stride = static_cast<uint32_t>(n_kv) * TILE;  // < 2^32 halves
  // Block ids of a step: one 16-byte scalar load while the step's 4 entries
  // lie in the table (each clamped into it otherwise; entries past the
  // sequence are never used).
  auto read_ids = [&](int (&ids)[kStepBlocks], int step) {
    if ((step + 1) * kStepBlocks <= table_len) {
      typedef int i32x4 __attribute__((ext_vector_type(4)));
      typedef const i32x4 __attribute__((address_space(4)))* const_i4_ptr;
      const i32x4 v = ((const_i4_ptr)table)[step];
      ids[0] = v.x;
      ids[1] = v.y;
      ids[2] = v.z;
      ids[3] = v.w;
    } else {
#pragma unroll
      for (int i = 0; i < kStepBlocks; ++i)
        ids[i] = scalar_load(table, min(step * kStepBlocks + i, table_len - 1));
    }
  };
  // halves from the pool's start to tile u's (block, kv head) tile; an id
  // outside the pool is reported and read as block 0
  auto tile_of = [&](const int (&ids)[kStepBlocks], int u) {
    int pb = ids[u * TPB + tsub];
    const bool ok = static_cast<uint32_t>(pb) < static_cast<uint32_t>(num_blocks);
    bad |= !ok;
    pb = ok ? pb : 0;
    return static_cast<int64_t>(static_cast<uint64_t>(static_cast<uint32_t>(pb)) * block_stride +
                                head_off);
  };
  typedef const void __attribute__((address_space(1)))* gptr_t;
  typedef void __attribute__((address_space(3)))* lptr_t;
  // Request step st's K (kv = 0) or V (kv = 1) tiles into buffer `buf`.
  auto issue = [&](const int (&ids)[kStepBlocks], int st, int buf, int kv) {
    f16* const d = lds.kv[buf][kv];
    const f16* const src = kv ? vp : kp;
    if ((st + 1) * kPfKeys <= seq_end) {
      // 4 whole blocks: straight into LDS, lane i's 16 bytes at base + 16 i
#pragma unroll
      for (int u = 0; u < KCH; ++u) {
        const int64_t tile = tile_of(ids, u);
        const int off = (u * TPB + tsub) * TILE + wchunk0 * 8;  // wave-uniform
        // the block's tile address held in scalar registers and the lane's
        // offset widened here (opaque copies), so that the load takes the
        // scalar-base form with a 32-bit per-lane offset
        const char* tb = reinterpret_cast<const char*>(src + tile);
        uint32_t lb = lane_byte;
        asm volatile("" : "+s"(tb), "+v"(lb));
        __builtin_amdgcn_global_load_lds((gptr_t)(tb + lb), (lptr_t)(d + off), 16, 0, 0);
      }
      return;
    }
    // the sequence's end: through registers, zeroing V past it (K past it is
    // masked out of the scores)
    const int key0 = st * kPfKeys;
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int bi = u * TPB + tsub;
      const int lb = key0 / kBlock + bi;
      f16x8 x = {0, 0, 0, 0, 0, 0, 0, 0};
      if (lb * kBlock < seq_end && lb < table_len) {
        const int64_t tile = tile_of(ids, u);
        x = *reinterpret_cast<const f16x8*>(src + tile + within * 8);
        if (kv) {
          // V chunk `within` holds slots 4q .. 4q+3 of two dims (tile order
          // [D/32][4][16][2][4])
          const int valid = seq_end - (lb * kBlock + ((within >> 4) & 3) * 4);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if ((e & 3) >= valid) x[e] = static_cast<f16>(0.0f);
        }
      }
      *reinterpret_cast<f16x8*>(d + bi * TILE + within * 8) = x;
    }
  };

  typedef f32x4 Scores[4][2];
  typedef f16x8 Probs[2][2];
  // S^T[key][M-row] = K . Q^T over the 4 blocks in K buffer `buf`.  Lane
  // (col, lg) reads K[slot col][dims 32kk + 8lg ..] of block mt, 16 bytes of
  // the tile order [D/8][16][8]: 1 KiB per wavefront and read.  Blocks go in
  // pairs: pair pr + 1's reads are requested before pair pr's products, which
  // then wait for pair pr's reads only (the scheduling fences keep that
  // order), and the two blocks' products interleave as four independent
  // accumulation chains (each still summing over kk in order).
  auto scores = [&](int buf, Scores& s) {
    const f16* const sk = lds.kv[buf][0] + lane * 8;
    f16x8 kb[2][2][KS];
    auto kload = [&](int pr, f16x8 (&dst)[2][KS]) {
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
          dst[e][kk] = *reinterpret_cast<const f16x8*>(sk + (2 * pr + e) * TILE + kk * 512);
    };
    kload(0, kb[0]);
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      if (pr + 1 < 2) kload(pr + 1, kb[(pr + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      f32x4 acc[2][2];
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[e][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
            acc[e][nt] = mfma16x16x32(kb[pr & 1][e][kk], qf[nt][kk], acc[e][nt]);
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) s[2 * pr + e][nt] = acc[e][nt];
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // causal mask of step `step`, only where it crosses the tile's diagonal
  auto mask = [&](int step, Scores& s) {
    const int key0 = step * kPfKeys;
    if (key0 + kPfKeys - 1 > q_start + r0) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int limit = q_start + min(mrow_r[nt], chunk_len - 1);  // last key allowed
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (key0 + mt * 16 + 4 * lg + j > limit) s[mt][nt][j] = -INFINITY;
      }
    }
  };
  // O^T[dim][M-row] += V^T[dim][key] . P^T[key][M-row]: lane (col, lg) of dim
  // tile dt, half h supplies dim 16dt + col at slots 4lg .. 4lg+3 of blocks 2h
  // and 2h + 1 (the keys the score accumulators give it).  In the tile order
  // [D/32][4][16][2][4] one 16-byte read per block holds that for dim tiles
  // 2p and 2p + 1; pair p + 1's reads are requested before pair p's products.
  auto pv = [&](int buf, const Probs& pb8) {
    const f16* const sv = lds.kv[buf][1] + lg * 128 + col * 8;
    f16x8 vb[2][4];
    auto vload = [&](int p, f16x8 (&dst)[4]) {
#pragma unroll
      for (int b = 0; b < 4; ++b) dst[b] = *reinterpret_cast<const f16x8*>(sv + b * TILE + p * 512);
    };
    vload(0, vb[0]);
#pragma unroll
    for (int p = 0; p < DT / 2; ++p) {
      if (p + 1 < DT / 2) vload(p + 1, vb[(p + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      const f16x8 (&r)[4] = vb[p & 1];
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const f16x8 va = {r[2 * h][4 * e], r[2 * h][4 * e + 1], r[2 * h][4 * e + 2],
                            r[2 * h][4 * e + 3], r[2 * h + 1][4 * e], r[2 * h + 1][4 * e + 1],
                            r[2 * h + 1][4 * e + 2], r[2 * h + 1][4 * e + 3]};
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
            o[2 * p + e][nt] = mfma16x16x32(va, pb8[h][nt], o[2 * p + e][nt]);
        }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int grp = wave >> 2;
  const int n = st1 - st0;
  int idK[kStepBlocks], idV[kStepBlocks];  // block ids of steps j + 1 and j
  Scores sc;
  Probs pb8;
  // product phase of step j (0 <= j <= n), at wave priority 1 so that its
  // products issue ahead of the other group's vector work
  auto products = [&](int j) {
    __builtin_amdgcn_s_setprio(1);
    if (j >= 1) pv((st0 + j - 1) & 1, pb8);
    if (j < n) scores((st0 + j) & 1, sc);
    __builtin_amdgcn_s_setprio(0);
  };
  // softmax phase of step j (0 <= j < n)
  auto softmax = [&](int j) {
    mask(st0 + j, sc);
    pf_softmax<DT>(sc, scale_log2, col, m_run, l_run, o, pb8);
  };
  // group 1's copies at phase 2j: K(j + 1) and V(j)
  auto copies = [&](int j) {
    if (j + 1 < n) issue(idK, st0 + j + 1, (st0 + j + 1) & 1, 0);
    if (j < n) issue(idV, st0 + j, (st0 + j) & 1, 1);
#pragma unroll
    for (int e = 0; e < kStepBlocks; ++e) idV[e] = idK[e];
    if (j + 2 < n) read_ids(idK, st0 + j + 2);
  };
  if (n > 0) {
    if (grp == 1) {
      read_ids(idV, st0);
      issue(idV, st0, st0 & 1, 0);
      if (n > 1) read_ids(idK, st0 + 1);
    }
    __builtin_amdgcn_s_waitcnt(kVmcnt0);  // this wavefront's copies into LDS have landed
    __syncthreads();
    // n + 1 rounds of two phases each; the two groups pass the same barriers
    if (grp == 0) {
      for (int j = 0; j <= n; ++j) {
        products(j);
        __syncthreads();
        if (j < n) softmax(j);
        __syncthreads();
      }
    } else {
      for (int j = 0; j <= n; ++j) {
        copies(j);
        if (j >= 1) softmax(j - 1);
        __syncthreads();
        products(j);
        __builtin_amdgcn_s_waitcnt(kVmcnt0);  // phase 2j's copies, before their readers
        __syncthreads();
      }
    }
  }

  if (bad) sbad = 1;
  __syncthreads();
  const bool any_bad = sbad != 0;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const float l = wave_sum_xor16_32(l_run[nt]);
    const int r = mrow_r[nt];
    if (r >= chunk_len) continue;
    const int head = g * G + mrow_h[nt];
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    const int64_t qh = static_cast<int64_t>(r) * n_q + head;
    if (splits == 1) {
      f16* orow = out + qh * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        f16x4 h4;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          h4[j] = static_cast<f16>(any_bad ? __builtin_nanf("") : o[dt][nt][j] * inv);
        *reinterpret_cast<f16x4*>(orow + dt * 16 + 4 * lg) = h4;
      }
    } else {
      const int64_t slot = static_cast<int64_t>(z) * chunk_len * n_q + qh;
      float* orow = a.ws_o + slot * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(orow + dt * 16 + 4 * lg) =
          o[dt][nt] * inv;
      if (lg == 0) {
        a.ws_m[slot] = any_bad ? __builtin_nanf("") : m_run[nt];
        a.ws_l[slot] = l;
      }
    }
  }
}

// Merge the key splits of (query row `row`, head `head`) by log-sum-exp; one
// wavefront, 64 threads.
template <int D>
__device__ __forceinline__ void prefill_reduce_row(int32_t chunk_len, int32_t n_q, int32_t splits,
                                                   const float* __restrict__ ws_o,
                                                   const float* __restrict__ ws_m,
                                                   const float* __restrict__ ws_l,
                                                   f16* __restrict__ out, int head, int row) {
  constexpr int PER = D / 64;
  constexpr int GRP = 4;  // splits whose partial rows are requested together
  const int lane = threadIdx.x;
  const int64_t qh = static_cast<int64_t>(row) * n_q + head;
  const int64_t stride = static_cast<int64_t>(chunk_len) * n_q;
  // split z's max and sum in lane z (splits <= 64), all requested at once
  // (lanes past the splits read split 0's and ignore it)
  const bool has = lane < splits;
  const int64_t zl = (has ? lane : 0) * stride + qh;
  const float m_in = ws_m[zl], l_in = ws_l[zl];
  const float mz = has ? m_in : -INFINITY;
  const float lz = has ? l_in : 0.0f;
  float M = -INFINITY;
  for (int z = 0; z < splits; ++z)
    M = fmaxf(M, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mz), z)));
  float wsum = 0.0f, acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.0f;
  for (int z0 = 0; z0 < splits; z0 += GRP) {
    float o[GRP][PER];
#pragma unroll
    for (int i = 0; i < GRP; ++i) {
      const int z = min(z0 + i, splits - 1);  // past the splits: the last one again, unused
      const float* op = ws_o + (z * stride + qh) * D;
#pragma unroll
      for (int e = 0; e < PER; ++e) o[i][e] = op[lane + 64 * e];
    }
#pragma unroll
    for (int i = 0; i < GRP; ++i) {
      const int z = z0 + i;
      if (z >= splits) break;
      const float m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mz), z));
      const float l = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lz), z));
      if (!(l > 0.0f) && !(m != m)) continue;
      const float w = l * exp2f(m - M);
      wsum += w;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] += w * o[i][e];
    }
  }
  const float inv = 1.0f / wsum;
  f16* orow = out + qh * D;
#pragma unroll
  for (int e = 0; e < PER; ++e) orow[lane + 64 * e] = static_cast<f16>(acc[e] * inv);
}


// Bytes of fp32 partials (o, m, l per split, row and head) the chunk needs;
// 0 when the key range is not split.
inline uint64_t prefill_ws_bytes(int32_t chunk_len, int32_t num_q_heads, int32_t head_dim,
                                 int32_t q_start) {
  if (chunk_len <= 0 || num_q_heads <= 0 || head_dim <= 0 || q_start < 0) return 0;
  const int s = prefill_splits(chunk_len, num_q_heads, q_start);
  if (s <= 1) return 0;
  return static_cast<uint64_t>(s) * chunk_len * num_q_heads * (head_dim + 2) * sizeof(float);
}

// Host checks of one chunk's arguments, then its kernel arguments and grid
// (kv head, query tile, key split).  PA_OK with chunk_len == 0 means there is
// nothing to launch.
inline pa_status prefill_prepare(pa_half* out, const pa_half* q, const pa_kv_view& kv,
                                 const int32_t* table, int32_t table_len, int32_t q_start,
                                 int32_t chunk_len, int32_t num_q_heads, float scale,
                                 void* workspace, uint64_t workspace_bytes, PrefillArgs& a,
                                 dim3& grid) {
  if (kv.k_pool == nullptr || kv.v_pool == nullptr || kv.block_size != kBlock ||
      kv.num_blocks <= 0 || kv.num_kv_heads <= 0 || kv.num_kv_heads > 65535)
    return PA_ERR_INVALID;
  if (kv.head_dim != 128 && kv.head_dim != 64) return PA_ERR_INVALID;
  if (q_start < 0 || chunk_len < 0 || table_len < 0) return PA_ERR_INVALID;
  if (num_q_heads <= 0 || num_q_heads % kv.num_kv_heads != 0) return PA_ERR_INVALID;
  const int G = num_q_heads / kv.num_kv_heads;
  if (G > 16 || kPfMRows % G != 0) return PA_ERR_INVALID;
  if (!scale_ok(scale)) return PA_ERR_INVALID;
  if (chunk_len == 0) return PA_OK;
  if (static_cast<int64_t>(q_start) + chunk_len > static_cast<int64_t>(table_len) * kBlock)
    return PA_ERR_INVALID;
  if (out == nullptr || q == nullptr || table == nullptr || !aligned16(q) || !aligned16(out) ||
      !aligned16(kv.k_pool) || !aligned16(kv.v_pool))
    return PA_ERR_INVALID;
  const int QR = kPfMRows / G;
  const int64_t qtiles = (static_cast<int64_t>(chunk_len) + QR - 1) / QR;
  if (qtiles > 65535) return PA_ERR_INVALID;
  const int splits = prefill_splits(chunk_len, num_q_heads, q_start);
  if (splits > 1 && chunk_len > 65535) return PA_ERR_INVALID;
  const int D = kv.head_dim;
  a.ws_o = a.ws_m = a.ws_l = nullptr;
  if (splits > 1) {
    const uint64_t need = prefill_ws_bytes(chunk_len, num_q_heads, D, q_start);
    if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace))
      return PA_ERR_INVALID;
    const int64_t slots = static_cast<int64_t>(splits) * chunk_len * num_q_heads;
    a.ws_o = static_cast<float*>(workspace);
    a.ws_m = a.ws_o + slots * D;
    a.ws_l = a.ws_m + slots;
  }
  a.q = reinterpret_cast<const f16*>(q);
  a.kp = reinterpret_cast<const f16*>(kv.k_pool);
  a.vp = reinterpret_cast<const f16*>(kv.v_pool);
  a.table = table;
  a.table_len = table_len;
  a.num_blocks = kv.num_blocks;
  a.n_kv = kv.num_kv_heads;
  a.G = G;
  a.q_start = q_start;
  a.chunk_len = chunk_len;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.splits = splits;
  a.out = reinterpret_cast<f16*>(out);
  grid = dim3(static_cast<uint32_t>(kv.num_kv_heads), static_cast<uint32_t>(qtiles),
              static_cast<uint32_t>(splits));
  return PA_OK;
}

}  // namespace pa
