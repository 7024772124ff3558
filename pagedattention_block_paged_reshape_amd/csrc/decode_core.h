// Paged decode attention on gfx950: device code (kernels, the work unit
// and merge helpers) and the host argument checks, shared by the decode
// launch (decode.hip) and the mixed decode + prefill launch (mixed.hip).
//
// What is computed (ta-paperlens "LLM serving from scratch", "fragmentation
// and PagedAttention": the attention kernel follows the logical-to-physical
// table and gathers K and V while it computes; media.tcdigital.jp, "logical
// and physical block mapping"): for request i, query head h, kv head
// g = h / G,
//     out[i][h] = sum_j softmax_j(scale * q[i][h] . K_j) * V_j,  j < len_i,
// token j living in physical block table[i][j/16], slot j%16.  Decode reads
// the whole cache once per step and does little arithmetic per byte
// (ta-paperlens, "prefill and decode"), so these kernels are built to stream
// the pool at HBM rate.
//
// Design (MI355X):
//  * Work unit = (kv head, request, partition of `part_blocks` blocks), done
//    by one workgroup of kDecodeWaves (2) wavefronts.  Two launch forms
//    share the code:
//      - grid form: one workgroup per unit, grid (kv head, request,
//        partition), empty units exit at once;
//      - work-list form (persistent): as many workgroups as stay resident;
//        each kv head's workgroups walk a host-built list of units, largest
//        first, dealt in snake order, so no workgroup launch sits between
//        units, the next unit's first block is in flight during a unit's
//        epilogue, and the last units to start are the small ones.
//    blockIdx.x is the kv head in both, so with 8 kv heads each head's
//    workgroups land on one XCD (workgroups are dealt to the 8 XCDs
//    round-robin), keeping that head's shared-prefix blocks in one L2.
//  * The G query heads that share a kv head are the 16 columns of a 16x16
//    MFMA tile (padded when G < 16), so each K/V byte is read once per kv
//    head, not once per query head.
//  * Each wavefront takes every other block of the unit.  A block's K tile
//    (16 tokens x D, 16*D*2 bytes contiguous, stored in MFMA operand order)
//    is loaded straight into the MFMA A-operand registers: S^T = K . Q^T
//    gives lane l the scores of 4 tokens for query head l%16.  Those scores,
//    after the online-softmax update, are already laid out as the B operand
//    of O^T += V^T . P^T, whose A operand is the V tile (also in operand
//    order).  Two register sets alternate so that one block's loads are in
//    flight while the other is computed; no LDS round trip in the main loop.
//  * Softmax runs in fp32 in base 2 (scores pre-multiplied by scale*log2 e);
//    the per-head running max is reduced across the 4 lane groups with the
//    gfx950 row-swap instructions, the running sum is kept per lane and
//    reduced at the end.
//  * The wavefronts merge through LDS with no closing barrier: each posts
//    its state and counts itself in; the last to arrive merges in fixed wave
//    order (deterministic) and stores.  A request that fits in one partition
//    gets its fp16 output directly; longer ones store an fp16 normalised
//    partial plus fp32 (max, sum), merged by the reduce kernel.
#pragma once

#include <math.h>

#include <stdlib.h>

#include <algorithm>

#include "pa_device.h"

namespace pa {

#ifndef PA_DECODE_WAVES
#define PA_DECODE_WAVES 2
#endif
#ifndef PA_MERGE_SLOTS
#define PA_MERGE_SLOTS 2
#endif
#ifndef PA_WL_WAVES_PER_EU
#define PA_WL_WAVES_PER_EU 2
#endif
constexpr int kDecodeWaves = PA_DECODE_WAVES;  // wavefronts per workgroup
constexpr int kDecodeThreads = kDecodeWaves * kWave;
constexpr int kMergeSlots = PA_MERGE_SLOTS;    // LDS merge slots of the work-list form
constexpr int kMaxWaveBlocks = 128;            // block ids a wavefront holds (2 per lane)
constexpr int kSpinLimit = 1 << 22;  // default bound on the LDS slot wait (s_sleep rounds)
constexpr size_t kResultRingBytes = 16384;  // LDS for buffered unit results (work-list form)

struct DecodeArgs {
  const f16* q;
  const f16* kp;
  const f16* vp;
  const int32_t* tables;
  const int32_t* seq_lens;
  int32_t batch;       // requests in the batch; work entries naming others are skipped
  int32_t spin_limit;  // bound on the work-list kernel's LDS slot wait
  int32_t max_blocks;
  int32_t num_blocks;
  int32_t n_kv;
  int32_t G;
  float scale_log2;
  int32_t part_blocks;
  int32_t p_max;
  f16* out;
  f16* ws_o;    // [B][n_kv][p_max][G][D] fp16
  float* ws_m;  // [B][n_kv][p_max][G]
  float* ws_l;  // [B][n_kv][p_max][G]
  float v_scale;  // FP8 pools: the V scale, applied when a unit is normalised
};

// One wavefront's share of a unit: running max and sum per query head and
// the unnormalised O^T tile (o[c][j] = O^T[c*16 + 4*(lane/16) + j][lane%16]).
template <int D>
struct WaveState {
  float m;
  float l;
  f32x4 o[D / 16];
};

// A request's length, clamped to what the tables and the partition grid can
// hold; anything clamped marks the request bad (its outputs become NaN).
__device__ __forceinline__ int clamp_len(const DecodeArgs& a, int b, bool& bad) {
  int L = scalar_load(a.seq_lens, b);
  if (L < 0) {
    L = 0;
    bad = true;
  }
  if (L > a.max_blocks * kBlock) {
    L = a.max_blocks * kBlock;
    bad = true;
  }
  if (L > a.p_max * a.part_blocks * kBlock) {
    L = a.p_max * a.part_blocks * kBlock;
    bad = true;
  }
  return L;
}

// A work unit (request b, partition p) as one wavefront sees it: the
// partition's blocks kb0 + wave + kDecodeWaves*i, i < cnt, and their physical
// ids (lane j of my_pb / my_pb2 holds the id of the wave's block j / 64 + j;
// at most 128 of them, which bounds partition_size).  A unit the lengths do not contain (a work
// list built from other lengths) is run as empty and not stored.
struct Unit {
  int b;
  int p;
  int L;        // attended length (0 for an empty or absent unit)
  int n_parts;  // partitions of the request
  int kb0;
  int cnt;
  int my_pb;   // id of the wave's block lane (lane < 64)
  int my_pb2;  // id of the wave's block 64 + lane
  bool ok;
  bool bad;
};

__device__ __forceinline__ Unit no_unit() {
  Unit u;
  u.b = u.p = u.L = u.n_parts = u.kb0 = u.cnt = u.my_pb = u.my_pb2 = 0;
  u.ok = false;
  u.bad = false;
  return u;
}

// Request b, partition p of a work entry (request << 16 | partition), or
// false when the entry names no unit of these lengths (request >= batch, or
// a partition the request does not have).  n_parts: the request's
// partitions (clamped as make_unit clamps them).
__device__ __forceinline__ bool entry_unit(const DecodeArgs& a, uint32_t packed, int& b, int& p,
                                           int& n_parts) {
  b = static_cast<int>(packed >> 16);
  p = static_cast<int>(packed & 0xFFFFu);
  if (b >= a.batch) return false;
  bool bad = false;
  const int L = clamp_len(a, b, bad);
  const int part_tokens = a.part_blocks * kBlock;
  n_parts = (L + part_tokens - 1) / part_tokens;
  return L > 0 ? p < n_parts : p == 0;
}

__device__ __forceinline__ Unit make_unit(const DecodeArgs& a, int b, int p, int wave, int lane) {
  Unit u;
  u.b = b;
  u.p = p;
  u.bad = false;
  const int L = clamp_len(a, b, u.bad);
  const int part_tokens = a.part_blocks * kBlock;
  u.n_parts = (L + part_tokens - 1) / part_tokens;
  u.ok = L > 0 ? p < u.n_parts : p == 0;
  u.L = u.ok ? L : 0;
  u.kb0 = (u.ok ? p : 0) * a.part_blocks;
  const int kb_end = min(u.kb0 + a.part_blocks, (u.L + kBlock - 1) / kBlock);
  const int nb = max(kb_end - u.kb0, 0);
  u.cnt = nb > wave ? (nb - wave + kDecodeWaves - 1) / kDecodeWaves : 0;
  // All of these are wave-uniform; saying so keeps the block loop's control
  // flow and block addresses in scalar registers.
  u.b = uniform(u.b);
  u.p = uniform(u.p);
  u.L = uniform(u.L);
  u.n_parts = uniform(u.n_parts);
  u.kb0 = uniform(u.kb0);
  u.cnt = uniform(u.cnt);
  const int32_t* trow = a.tables + static_cast<int64_t>(b) * a.max_blocks;
  u.my_pb = 0;
  u.my_pb2 = 0;
  auto fetch_id = [&](int j, int& dst) {
    if (j < u.cnt) {
      const int pb = trow[u.kb0 + wave + kDecodeWaves * j];
      if (static_cast<uint32_t>(pb) < static_cast<uint32_t>(a.num_blocks))
        dst = pb;
      else
        u.bad = true;  // replaced by block 0; the request's output becomes NaN
    }
  };
  fetch_id(lane, u.my_pb);
  if (u.cnt > kWave) fetch_id(kWave + lane, u.my_pb2);
  return u;
}


// The unit of a work entry (request << 16 | partition).  An entry naming a
// request outside the batch (a list built for other lengths) becomes
// request 0's partition 65535, which no request has: an empty unit that is
// not stored (the choice is made on the scalars, which costs no registers).
__device__ __forceinline__ Unit make_entry_unit(const DecodeArgs& a, uint32_t packed, int wave,
                                                int lane) {
  const bool in_batch = static_cast<int>(packed >> 16) < a.batch;
  return make_unit(a, in_batch ? static_cast<int>(packed >> 16) : 0,
                   in_batch ? static_cast<int>(packed & 0xFFFFu) : 0xFFFF, wave, lane);
}

// Q^T as the B operand: lane holds query head lane%16 (zero when >= G), dims
// kk*32 + 8*(lane/16) .. +8.
template <int D>
__device__ __forceinline__ void load_q(const DecodeArgs& a, int g, int b, int lane, f16x8* qf) {
  const int col = lane & 15;
  const int lg = lane >> 4;
  const f16* qrow =
      a.q + (static_cast<int64_t>(b) * a.n_kv * a.G + g * a.G + col) * D + lg * 8;
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk)
    qf[kk] = col < a.G ? *reinterpret_cast<const f16x8*>(qrow + kk * 32)
                       : f16x8{0, 0, 0, 0, 0, 0, 0, 0};
}

// K and V tiles of physical block pb, kv head g, straight into MFMA operand
// registers.  The tiles are stored in operand order, so each load is 16 B
// per lane with lane i on bytes [16i, 16i+16) of a 1 KiB span:
//   K step kk: lane l gets K[slot l%16][dims kk*32 + 8*(l/16) .. +8];
//   V pair cc: lane l gets V[slots 4*(l/16) .. +4][dim (2cc+h)*16 + l%16] for
//   h = 0, 1, i.e. the A operands of dim tiles 2cc and 2cc+1.
// Unless KEEP, the loads are non-temporal: a tile is read once per launch
// when no two requests share it, and streaming it keeps it from competing
// for cache lines with the tables, queries and partials (on the
// Llama-3-70B-shaped layer this alone took the launch from ~262 us to
// ~233 us, 5.4 -> 6.0 TB/s).  When requests share blocks (a common prefix),
// KEEP loads them normally so that the shared tiles stay in L2.
template <int D, bool KEEP>
__device__ __forceinline__ f16x8 load_tile16(const f16* p) {
  const f16x8* q = reinterpret_cast<const f16x8*>(p);
  return KEEP ? *q : __builtin_nontemporal_load(q);
}

template <bool KEEP>
__device__ __forceinline__ u32x4 load_bytes16(const uint8_t* p) {
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
  return KEEP ? *q : __builtin_nontemporal_load(q);
}

// One block's operand registers: K[NK] and V[NV]; a register set holds NB
// blocks.  fp16 tiles load straight into the MFMA operands; FP8 tiles load as
// bytes (half the registers) and are widened when computed, and a set holds
// two blocks, so that a wavefront keeps as many bytes in flight as with fp16.
template <int D, bool FP8>
struct TileRegs {
  typedef f16x8 K;
  typedef f16x4 V;
  static constexpr int NK = D / 32;
  static constexpr int NV = D / 16;
  static constexpr int NB = 1;
};
template <int D>
struct TileRegs<D, true> {
  typedef u32x4 K;  // bytes [16 lane, 16 lane + 16) of each 1 KiB K span
  typedef u32x4 V;
  static constexpr int NK = D / 64;
  static constexpr int NV = D / 64;
  static constexpr int NB = 2;
};

template <int D, bool KEEP, bool FP8>
__device__ __forceinline__ void load_block(const DecodeArgs& a, int g, int pb, int lane,
                                           typename TileRegs<D, FP8>::K* kd,
                                           typename TileRegs<D, FP8>::V* vd) {
  const int64_t tile = (static_cast<int64_t>(pb) * a.n_kv + g) * (kBlock * D);  // uniform
  if constexpr (FP8) {
    // tile in bytes: lane i reads bytes [16i, 16i + 16) of each 1 KiB span
    const uint8_t* kt = reinterpret_cast<const uint8_t*>(a.kp) + tile + lane * 16;
    const uint8_t* vt = reinterpret_cast<const uint8_t*>(a.vp) + tile + lane * 16;
#pragma unroll
    for (int p = 0; p < D / 64; ++p) kd[p] = load_bytes16<KEEP>(kt + p * 1024);
#pragma unroll
    for (int p = 0; p < D / 64; ++p) vd[p] = load_bytes16<KEEP>(vt + p * 1024);
  } else {
    const f16* kt = a.kp + tile + lane * 8;
    const f16* vt = a.vp + tile + lane * 8;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
      kd[kk] = load_tile16<D, KEEP>(kt + kk * 512);
#pragma unroll
    for (int cc = 0; cc < D / 32; ++cc) {
      const f16x8 pair = load_tile16<D, KEEP>(vt + cc * 512);
      vd[2 * cc] = f16x4{pair[0], pair[1], pair[2], pair[3]};
      vd[2 * cc + 1] = f16x4{pair[4], pair[5], pair[6], pair[7]};
    }
  }
}

// Four E4M3 codes (byte j of w is element j) as fp16.  Every E4M3 value is
// exact in fp16, so with a unit scale the conversion is exact.
__device__ __forceinline__ f16x4 e4m3x4_to_f16(uint32_t w) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 r = {
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true))};
  return __builtin_bit_cast(f16x4, r);
}

// FP8 block registers as the fp16 operands load_block gives for fp16 tiles:
// load p's dwords 0-1 / 2-3 are K steps 2p / 2p+1; its dword t is V dim tile
// 4p + t.
template <int D>
__device__ __forceinline__ void widen(const u32x4* kr, const u32x4* vr, f16x8* kf, f16x4* vf) {
#pragma unroll
  for (int p = 0; p < D / 64; ++p) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f16x4 lo = e4m3x4_to_f16(kr[p][2 * h]);
      const f16x4 hi = e4m3x4_to_f16(kr[p][2 * h + 1]);
      kf[2 * p + h] = f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) vf[4 * p + t] = e4m3x4_to_f16(vr[p][t]);
  }
}

// Physical block behind the wave's i-th load (slot s of its register set):
// unit u's blocks first; past them the next unit's block s (so that it is in
// flight during u's epilogue), or, when there is none or `zero` is set,
// block 0: one tile that every such stand-in load shares, so it stays cached
// (the loads are non-temporal, so re-reading u's last block would go to HBM
// again).
__device__ __forceinline__ int unit_block(const Unit& u, int i) {
  return i < kWave ? __builtin_amdgcn_readlane(u.my_pb, i)
                   : __builtin_amdgcn_readlane(u.my_pb2, i - kWave);
}

__device__ __forceinline__ int pick_block(const Unit& u, const Unit& nx, int i, int s = 0,
                                          bool zero = false) {
  int pb;
  if (i < u.cnt)
    pb = unit_block(u, i);
  else if (!zero && nx.cnt > s)
    pb = unit_block(nx, s);
  else
    pb = 0;
  return uniform(pb);
}

// Load register set (ks, vs) with the wave's blocks j0 .. j0 + NB - 1 of u.
// A set that carries over to the next unit (`carry`, and entirely past u's
// end) takes nx's first NB blocks; any other stand-in of a two-block set
// reads block 0, so that no block is fetched twice.
template <int D, bool KEEP, bool FP8>
__device__ __forceinline__ void load_set(const DecodeArgs& a, int g, const Unit& u,
                                         const Unit& nx, int j0, bool carry, int lane,
                                         typename TileRegs<D, FP8>::K* ks,
                                         typename TileRegs<D, FP8>::V* vs) {
  typedef TileRegs<D, FP8> TR;
#pragma unroll
  for (int s = 0; s < TR::NB; ++s) {
    const bool zero = TR::NB > 1 && !(carry && j0 >= u.cnt);
    load_block<D, KEEP, FP8>(a, g, pick_block(u, nx, j0 + s, s, zero), lane, ks + s * TR::NK,
                             vs + s * TR::NV);
  }
}

// The wavefront's pass over its blocks of unit u on kv head g.  On entry
// kA/vA hold u's first NB blocks (when u.cnt > 0); on exit they hold nx's
// first NB blocks (when nx.cnt > 0).
template <int D, bool KEEP, bool FP8>
__device__ __forceinline__ void run_unit(const DecodeArgs& a, int g, int wave, int lane,
                                         const Unit& u, const Unit& nx, const f16x8* qf,
                                         typename TileRegs<D, FP8>::K* kA,
                                         typename TileRegs<D, FP8>::V* vA,
                                         typename TileRegs<D, FP8>::K* kB,
                                         typename TileRegs<D, FP8>::V* vB, WaveState<D>& st) {
  constexpr int KS = D / 32;  // K-steps of the score MFMA
  constexpr int DT = D / 16;  // 16-wide dimension tiles of the output
  const int lg = lane >> 4;   // lane group: which 8 (K) or 4 (V, P) k-values

  st.m = -INFINITY;
  st.l = 0.0f;
#pragma unroll
  for (int c = 0; c < DT; ++c) st.o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (u.cnt == 0) {
    if (nx.cnt > 0) load_set<D, KEEP, FP8>(a, g, u, nx, 0, true, lane, kA, vA);
    return;
  }
  const int L = u.L;

  // Online-softmax update with the wave's i-th block.
  auto compute = [&](int i, const f16x8* kf, f16x4* vf) {
    const int kb = u.kb0 + wave + kDecodeWaves * i;
    // S^T tile: lane gets tokens kb*16 + 4*lg + j for query head lane%16.
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) s = mfma16x16x32(kf[kk], qf[kk], s);
    const int tok0 = kb * kBlock + 4 * lg;
    const int valid = L - tok0;  // this lane's tokens j < valid are live
    float sv[4];
    float mloc = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sv[j] = j < valid ? s[j] * a.scale_log2 : -INFINITY;
      mloc = fmaxf(mloc, sv[j]);
    }
    mloc = wave_max_xor16_32(mloc);
    const float m_new = fmaxf(st.m, mloc);
    // hardware 2^x: results below 2^-126 flush to 0, which softmax ignores
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
    f16x4 pf;
    float psum = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f16 ph = static_cast<f16>(__builtin_amdgcn_exp2f(sv[j] - m_new));
      pf[j] = ph;
      psum += static_cast<float>(ph);
    }
    st.l = st.l * alpha + psum;
    st.m = m_new;
    if ((kb + 1) * kBlock > L) {
      // The request's last block: slots past its end hold stale bytes; clear
      // them so that 0 * stale cannot inject NaN/Inf into the MFMA.
      const uint32_t lo = valid >= 2 ? 0xFFFFFFFFu : (valid == 1 ? 0x0000FFFFu : 0u);
      const uint32_t hi = valid >= 4 ? 0xFFFFFFFFu : (valid == 3 ? 0x0000FFFFu : 0u);
#pragma unroll
      for (int c = 0; c < DT; ++c) {
        uint2 bits = __builtin_bit_cast(uint2, vf[c]);
        bits.x &= lo;
        bits.y &= hi;
        vf[c] = __builtin_bit_cast(f16x4, bits);
      }
    }
    // Rescale only when some head's running max moved (alpha != 1).
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
      for (int c = 0; c < DT; ++c) st.o[c] *= alpha;
    }
#pragma unroll
    for (int c = 0; c < DT; ++c) st.o[c] = mfma16x16x16(vf[c], pf, st.o[c]);
  };

  // FP8 tiles are widened to fp16 first (K's scale is folded into
  // scale_log2, V's into the final normalisation).
  auto step = [&](int i, typename TileRegs<D, FP8>::K* kr, typename TileRegs<D, FP8>::V* vr) {
    if constexpr (FP8) {
      f16x8 kf[KS];
      f16x4 vf[DT];
      widen<D>(kr, vr, kf, vf);
      compute(i, kf, vf);
    } else {
      compute(i, kr, vr);
    }
  };

  // Two register sets in ping-pong: while one set's blocks are computed the
  // other's loads are in flight; no register copies, so the compiler's wait
  // counts only cover the blocks being consumed.  Every load is
  // unconditional (pick_block), the last one into kA/vA being nx's first.
  typedef TileRegs<D, FP8> TR;
  constexpr int NB = TR::NB;
  for (int i = 0; i < u.cnt; i += 2 * NB) {
    load_set<D, KEEP, FP8>(a, g, u, nx, i + NB, false, lane, kB, vB);
#pragma unroll
    for (int s = 0; s < NB; ++s)
      if (s == 0 || i + s < u.cnt) step(i + s, kA + s * TR::NK, vA + s * TR::NV);
    load_set<D, KEEP, FP8>(a, g, u, nx, i + 2 * NB, true, lane, kA, vA);
#pragma unroll
    for (int s = 0; s < NB; ++s)
      if (i + NB + s < u.cnt) step(i + NB + s, kB + s * TR::NK, vB + s * TR::NV);
  }
}

// LDS of one merge: per-wave (m, l) per head and O^T rows [wave][head][D+4].
template <int D>
struct MergeSlot {
  float* m;  // [kDecodeWaves][16]
  float* l;  // [kDecodeWaves][16]
  float* o;  // [kDecodeWaves][G][D + 4]
  int* arrive;
  int* bad;
};

// Post the wave's state; returns true for the last of the kDecodeWaves
// wavefronts to arrive.
template <int D>
__device__ __forceinline__ bool post_state(const MergeSlot<D>& ms, const WaveState<D>& st, int G,
                                           int wave, int lane, bool bad) {
  constexpr int DT = D / 16;
  constexpr int OROW = D + 4;
  const int col = lane & 15;
  const int lg = lane >> 4;
  const float l = wave_sum_xor16_32(st.l);
  if (lg == 0) {
    ms.m[wave * 16 + col] = st.m;
    ms.l[wave * 16 + col] = l;
  }
  if (col < G) {
    float* row = ms.o + (wave * G + col) * OROW + 4 * lg;
#pragma unroll
    for (int c = 0; c < DT; ++c) *reinterpret_cast<f32x4*>(row + c * 16) = st.o[c];
  }
  if (bad) __hip_atomic_store(ms.bad, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  int arrived = 0;
  if (lane == 0)
    arrived = __hip_atomic_fetch_add(ms.arrive, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
  arrived = __shfl(arrived, 0);
  return arrived == kDecodeWaves - 1;
}

// Merge the posted states of a unit in fixed wave order: each lane produces
// 8 consecutive dims of one head and hands them, with the head's running max
// and sum, to emit(h, d0, r, m, l).  An empty request reads as zeros, a
// flagged one as NaN.  FP8 pools scale the normalised rows by v_scale.
template <int D, bool FP8, typename Emit>
__device__ __forceinline__ void merge_unit(const MergeSlot<D>& ms, int G, int L, int lane,
                                           float v_scale, Emit emit) {
  constexpr int OROW = D + 4;
  const bool any_bad =
      __hip_atomic_load(ms.bad, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0;
  for (int idx = lane; idx < G * (D / 8); idx += kWave) {
    const int h = idx / (D / 8);
    const int d0 = (idx % (D / 8)) * 8;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) M = fmaxf(M, ms.m[w * 16 + h]);
    float wsum = 0.0f;
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
    if (L > 0) {
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w) {
        const float e = exp2f(ms.m[w * 16 + h] - M);
        wsum += e * ms.l[w * 16 + h];
        const float* row = ms.o + (w * G + h) * OROW + d0;
        a0 += e * *reinterpret_cast<const f32x4*>(row);
        a1 += e * *reinterpret_cast<const f32x4*>(row + 4);
      }
    }
    const float inv =
        any_bad ? __builtin_nanf("") : (L > 0 ? (FP8 ? v_scale / wsum : 1.0f / wsum) : 0.0f);
    f16x8 r;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      r[k] = static_cast<f16>(a0[k] * inv);
      r[k + 4] = static_cast<f16>(a1[k] * inv);
    }
    emit(h, d0, r, any_bad ? __builtin_nanf("") : M, wsum);
  }
}

// Global destination of a unit's merged rows: the request's output rows if
// it has one partition, else its partial slot ([B][n_kv][p_max][G][D] fp16,
// (m, l) as [B][n_kv][p_max][G] fp32).
template <int D>
__device__ __forceinline__ void store_rows(const DecodeArgs& a, int g, int b, int p,
                                           int n_parts, int h, int d0, f16x8 r, float m,
                                           float l) {
  // Output rows: streaming (non-temporal) stores, since nothing on the GPU
  // reads them back.  Partials: plain stores, since the reduce launch that
  // follows reads them, on the same XCD (both grids put kv head g there);
  // measured on the Llama-3-70B-shaped layer, 240.3 vs 243.2 us per launch.
  const int G = a.G;
  if (n_parts <= 1) {
    const int64_t qh = static_cast<int64_t>(b) * a.n_kv * G + g * G + h;
    __builtin_nontemporal_store(r, reinterpret_cast<f16x8*>(a.out + qh * D + d0));
  } else {
    const int64_t slot = ((static_cast<int64_t>(b) * a.n_kv + g) * a.p_max + p) * G + h;
    *reinterpret_cast<f16x8*>(a.ws_o + slot * D + d0) = r;
    if (d0 == 0) {
      a.ws_m[slot] = m;
      a.ws_l[slot] = l;
    }
  }
}

template <int D, bool FP8>
__device__ __forceinline__ void merge_store(const DecodeArgs& a, const MergeSlot<D>& ms, int g,
                                            int b, int p, int L, int n_parts, int lane) {
  merge_unit<D, FP8>(ms, a.G, L, lane, a.v_scale, [&](int h, int d0, f16x8 r, float m, float l) {
    store_rows<D>(a, g, b, p, n_parts, h, d0, r, m, l);
  });
}

// Merge the partial states of partitions [p_begin, p_end) of one (request,
// query head) over the 8 * NV dims from d0: with M = max_p m_p and
// w_p = l_p * 2^(m_p - M), acc = sum_p w_p o_p and wsum = sum_p w_p, the sums
// taken in partition order (each partition's exp sum rescaled to the common
// max, which gives exactly the softmax over those partitions' tokens;
// acc / wsum is the merged output).  `bg` is the (request, kv head)'s first
// partial slot.  The partials of up to kChunk partitions are requested at
// once, so a range of up to kChunk partitions costs one memory round trip.
// An empty range gives M = -inf, wsum = 0, acc = 0.
template <int D, int NV>
__device__ __forceinline__ void merge_range(const DecodeArgs& a, int64_t bg, int h, int d0,
                                            int p_begin, int p_end, float& M, float& wsum,
                                            float (&acc)[NV][8]) {
  constexpr int kChunk = 8;
  const int G = a.G;
  f16x8 v[kChunk][NV];
  float mm[kChunk], ll[kChunk];
  auto load = [&](int p0) {
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      if (p0 + u < p_end) {
        const int64_t slot = bg + static_cast<int64_t>(p0 + u) * G + h;
#pragma unroll
        for (int c = 0; c < NV; ++c)
          v[u][c] = *reinterpret_cast<const f16x8*>(a.ws_o + slot * D + d0 + 8 * c);
        mm[u] = a.ws_m[slot];
        ll[u] = a.ws_l[slot];
      }
    }
  };
  load(p_begin);
  M = -INFINITY;
#pragma unroll
  for (int u = 0; u < kChunk; ++u)
    if (p_begin + u < p_end) M = fmaxf(M, mm[u]);
  for (int p = p_begin + kChunk; p < p_end; ++p)
    M = fmaxf(M, a.ws_m[bg + static_cast<int64_t>(p) * G + h]);
  wsum = 0.0f;
#pragma unroll
  for (int c = 0; c < NV; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[c][e] = 0.0f;
  for (int p0 = p_begin; p0 < p_end; p0 += kChunk) {
    if (p0 > p_begin) load(p0);
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      if (p0 + u < p_end) {
        const float w = ll[u] * exp2f(mm[u] - M);
        wsum += w;
#pragma unroll
        for (int c = 0; c < NV; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[c][e] += w * static_cast<float>(v[u][c][e]);
      }
    }
  }
}

// Second kernel of both launch forms: one workgroup per (kv head, request)
// merges the request's partitions, D/16 lanes per query head and 16 dims
// per lane.  The kernel is bound by memory latency: it reads the request's
// length, then the partials, kChunk partitions per round trip.  With one
// wavefront (requests of up to a few partitions) that lane merges all of
// them.  With W = blockDim.x / 64 > 1 wavefronts (long requests), wavefront
// w merges the contiguous range [w*P/W, (w+1)*P/W) of the P partitions, and
// the W states (M_w, wsum_w, acc_w) are combined through LDS in wavefront
// order: M = max M_w, out = sum_w acc_w 2^(M_w - M) / sum_w wsum_w 2^(M_w - M).
// Requests that fit in one partition were written by the first kernel and
// are skipped.  A NaN-flagged partial makes the output NaN either way.
constexpr int kReduceMaxWaves = 4;
constexpr int kReduceWideParts = 16;  // requests of at least this many partitions use 4 waves
constexpr int kReduceEntry = 18;      // floats per combine entry: M, wsum, 16 accumulators

template <int D>
__device__ __forceinline__ void decode_reduce_unit(const DecodeArgs& a, int g, int b) {
  constexpr int LPH = D / 16;  // lanes per query head
  // dynamic LDS (W > 1 only): [W][G * LPH][kReduceEntry] floats
  extern __shared__ f32x4 sm_o4[];
  float* const red = reinterpret_cast<float*>(sm_o4);
  const int G = a.G;
  const int W = blockDim.x / kWave;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int part_tokens = a.part_blocks * kBlock;
  int L = scalar_load(a.seq_lens, b);
  if (L < 0) return;                                         // written as NaN already
  if (L > a.max_blocks * kBlock) L = a.max_blocks * kBlock;  // partials are NaN-flagged
  const int n_parts = min((L + part_tokens - 1) / part_tokens, a.p_max);
  if (n_parts <= 1) return;
  const int64_t bg = (static_cast<int64_t>(b) * a.n_kv + g) * a.p_max * G;
  const int p0 = wave * n_parts / W;
  const int p1 = (wave + 1) * n_parts / W;
  for (int idx = lane; idx < G * LPH; idx += kWave) {
    const int h = idx / LPH;
    const int d0 = (idx % LPH) * 16;
    float M, wsum, acc[2][8];
    merge_range<D, 2>(a, bg, h, d0, p0, p1, M, wsum, acc);
    if (W == 1) {
      const float inv = 1.0f / wsum;
      f16x8 r[2];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) r[c][e] = static_cast<f16>(acc[c][e] * inv);
      f16* dst = a.out + ((static_cast<int64_t>(b) * a.n_kv + g) * G + h) * D + d0;
      *reinterpret_cast<f16x8*>(dst) = r[0];
      *reinterpret_cast<f16x8*>(dst + 8) = r[1];
    } else {
      float* e = red + (wave * G * LPH + idx) * kReduceEntry;
      e[0] = M;
      e[1] = wsum;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int k = 0; k < 8; ++k) e[2 + 8 * c + k] = acc[c][k];
    }
  }
  if (W == 1) return;
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * LPH; idx += blockDim.x) {
    const int h = idx / LPH;
    const int d0 = (idx % LPH) * 16;
    float M = -INFINITY;
    for (int w = 0; w < W; ++w) M = fmaxf(M, red[(w * G * LPH + idx) * kReduceEntry]);
    float wsum = 0.0f, acc[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[k] = 0.0f;
    for (int w = 0; w < W; ++w) {
      const float* e = red + (w * G * LPH + idx) * kReduceEntry;
      const float s = exp2f(e[0] - M);
      wsum += e[1] * s;
#pragma unroll
      for (int k = 0; k < 16; ++k) acc[k] += e[2 + k] * s;
    }
    const float inv = 1.0f / wsum;
    f16x8 r[2];
#pragma unroll
    for (int k = 0; k < 16; ++k) r[k / 8][k % 8] = static_cast<f16>(acc[k] * inv);
    f16* dst = a.out + ((static_cast<int64_t>(b) * a.n_kv + g) * G + h) * D + d0;
    *reinterpret_cast<f16x8*>(dst) = r[0];
    *reinterpret_cast<f16x8*>(dst + 8) = r[1];
  }
}

template <int D>
__global__ __launch_bounds__(kReduceMaxWaves * kWave) void decode_reduce_kernel(DecodeArgs a) {
  decode_reduce_unit<D>(a, blockIdx.x, blockIdx.y);
}

// Wavefronts per reduce workgroup for a batch whose longest request has
// p_max partitions, and the dynamic LDS that takes.
inline int reduce_waves(int p_max) { return p_max >= kReduceWideParts ? kReduceMaxWaves : 1; }
inline size_t reduce_lds(int p_max, int G, int D) {
  const int W = reduce_waves(p_max);
  return W > 1 ? static_cast<size_t>(W) * G * (D / 16) * kReduceEntry * sizeof(float) : 0;
}

// Grid form: one workgroup per (kv head, request, partition).
template <int D, bool KEEP, bool FP8>
__global__ __launch_bounds__(kDecodeThreads) void decode_partition_kernel(DecodeArgs a) {
  const int g = blockIdx.x;
  const int b = blockIdx.y;
  const int p = blockIdx.z;
  bool bad = false;
  const int L = clamp_len(a, b, bad);
  const int part_tokens = a.part_blocks * kBlock;
  const int n_parts = (L + part_tokens - 1) / part_tokens;
  if (L > 0 ? p >= n_parts : p > 0) return;

  __shared__ float sm_m[kDecodeWaves * 16];
  __shared__ float sm_l[kDecodeWaves * 16];
  __shared__ int sm_arrive;
  __shared__ int sm_bad;
  extern __shared__ f32x4 sm_o4[];  // [kDecodeWaves][G][D + 4] floats, 16-byte aligned
  if (threadIdx.x == 0) {
    sm_arrive = 0;
    sm_bad = 0;
  }
  __syncthreads();

  const int wave = uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const Unit u = make_unit(a, b, p, wave, lane);
  const Unit nx = no_unit();
  typedef TileRegs<D, FP8> TR;
  f16x8 qf[D / 32];
  typename TR::K kA[TR::NB * TR::NK], kB[TR::NB * TR::NK];
  typename TR::V vA[TR::NB * TR::NV], vB[TR::NB * TR::NV];
  if (u.cnt > 0) {
    load_q<D>(a, g, b, lane, qf);
    load_set<D, KEEP, FP8>(a, g, u, nx, 0, true, lane, kA, vA);
  }
  WaveState<D> st;
  run_unit<D, KEEP, FP8>(a, g, wave, lane, u, nx, qf, kA, vA, kB, vB, st);
  const MergeSlot<D> ms{sm_m, sm_l, reinterpret_cast<float*>(sm_o4), &sm_arrive, &sm_bad};
  if (post_state<D>(ms, st, a.G, wave, lane, u.bad))
    merge_store<D, FP8>(a, ms, g, b, p, u.L, n_parts, lane);
}

// LDS of one wavefront pair's work-list walk: kMergeSlots merge slots (per
// wavefront and head the running max and sum, and the O^T rows), their
// arrival, bad and merged counters, the pair's give-up flag, and the result
// ring of `ring` units: (request, partition, partitions, valid), the fp16
// rows, and each row's max and sum.
struct WalkLds {
  float* m;          // [kMergeSlots][kDecodeWaves * 16]
  float* l;          // [kMergeSlots][kDecodeWaves * 16]
  int* arrive;       // [kMergeSlots]
  int* bad;          // [kMergeSlots]
  int* merged;       // [kMergeSlots]
  int* abandon;      // one flag
  float* o;          // [kMergeSlots][kDecodeWaves][G][D + 4]
  int4* ring_info;   // [ring]
  f16* ring_o;       // [ring][G][D]
  float* ring_m;     // [ring][G]
  float* ring_l;     // [ring][G]
};

// Bytes of the merge states and of one result-ring unit, for G query heads.
__host__ __device__ constexpr size_t walk_merge_bytes(int G, int D) {
  return static_cast<size_t>(kMergeSlots) * kDecodeWaves * G * (D + 4) * sizeof(float);
}
__host__ __device__ constexpr size_t walk_ring_slot_bytes(int G, int D) {
  return static_cast<size_t>(G) * D * 2 + 2 * G * sizeof(float) + 16;
}
// One pair's whole LDS as walk_carve lays it out, a multiple of 16 bytes.
__host__ __device__ constexpr size_t walk_pair_bytes(int G, int D, int ring) {
  return (walk_merge_bytes(G, D) + 2 * kMergeSlots * kDecodeWaves * 16 * sizeof(float) +
          16 * ((3 * kMergeSlots + 1 + 3) / 4) + ring * walk_ring_slot_bytes(G, D) + 15) /
         16 * 16;
}

// A pair's WalkLds carved from `base` (16-byte aligned), in walk_pair_bytes'
// layout: merge rows, max, sum, counters, ring info, ring rows, ring max, sum.
template <int D>
__device__ __forceinline__ WalkLds walk_carve(char* base, int G, int ring) {
  WalkLds w;
  char* p = base;
  w.o = reinterpret_cast<float*>(p);
  p += walk_merge_bytes(G, D);
  w.m = reinterpret_cast<float*>(p);
  p += kMergeSlots * kDecodeWaves * 16 * sizeof(float);
  w.l = reinterpret_cast<float*>(p);
  p += kMergeSlots * kDecodeWaves * 16 * sizeof(float);
  w.arrive = reinterpret_cast<int*>(p);
  w.bad = w.arrive + kMergeSlots;
  w.merged = w.bad + kMergeSlots;
  w.abandon = w.merged + kMergeSlots;
  p += 16 * ((3 * kMergeSlots + 1 + 3) / 4);
  w.ring_info = reinterpret_cast<int4*>(p);
  w.ring_o = reinterpret_cast<f16*>(w.ring_info + ring);
  w.ring_m = reinterpret_cast<float*>(w.ring_o + ring * G * D);
  w.ring_l = w.ring_m + ring * G;
  return w;
}

// Units of the snake deal that pair y of wph gets from a list of n_items:
// every full round, and the last, partial one if it reaches y.
__device__ __forceinline__ int walk_units(int n_items, int wph, int y) {
  const int R = n_items / wph;
  const int rem = n_items % wph;
  const bool part = rem > 0 && ((R & 1) ? (wph - 1 - y) < rem : y < rem);
  return R + (part ? 1 : 0);
}

// The work-list walk of one wavefront pair: pair y of the wph pairs of kv
// head g walks `items` ((request << 16) | partition, largest first) in a
// snake deal: in round r pair y takes entry r*wph + y, reversed on odd
// rounds, which gives every pair a near-equal share of blocks and leaves the
// smallest units for last.  While a unit is computed the next unit's block
// ids are already loaded, and its first block and query rows are in flight
// during the unit's epilogue.  LDS merge slots rotate over consecutive units
// so that a fast wavefront can post the next unit while the last one of an
// earlier unit still merges.
//
// Merged results are not stored when a unit ends: they go to an LDS ring of
// `ring` unit slots, written to HBM when the ring is full and when the
// walk is done.  On this GPU a wavefront's stores and loads retire in order,
// so a store issued at a unit's end would make the next unit's first wait
// also wait for the store's acknowledgement; measured on the
// Llama-3-70B-shaped layer that cost ~8 % of the launch.
//
// With several pairs in a workgroup (MULTI), every pair runs k_end
// iterations (the most units any of them has; a pair past its own units runs
// empty ones), so the ring windows end at the same iterations everywhere and
// their barriers are the workgroup's; with one pair, k_end is unused and the
// walk ends with the pair's last unit.  The LDS counters must be zero on
// entry, behind a barrier.
template <int D, bool KEEP, bool FP8, bool MULTI>
__device__ __forceinline__ void worklist_walk(const DecodeArgs& a,
                                              const int32_t* __restrict__ items,
                                              int32_t n_items, int32_t ring, int g, int y,
                                              int wph, int k_end, int wave, int lane,
                                              const WalkLds& w) {
  const int G = a.G;
  const int slot_floats = kDecodeWaves * G * (D + 4);
  auto item = [&](int k) { return (k & 1) ? (k + 1) * wph - 1 - y : k * wph + y; };
  auto has = [&](int k) { return (!MULTI || k < k_end) && item(k) < n_items; };
  auto unit_at = [&](int t) {
    return make_entry_unit(a, static_cast<uint32_t>(scalar_load(items, t)), wave, lane);
  };
  // Give up on this pair's remaining work: mark it abandoned for the other
  // wavefront, then write NaN rows (and NaN max and sum) to the destination
  // of every unit of the deal from entry index k0 on.  Units before k0 were
  // flushed; the rest are in the LDS ring or not yet done, and which of
  // those are whole cannot be told, so all of them read as bad.  Both
  // wavefronts may do this; they write the same values.
  auto abandon = [&](int k0) {
    if (lane == 0)
      __hip_atomic_store(w.abandon, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    const float nan = __builtin_nanf("");
    const f16 hn = static_cast<f16>(nan);
    const f16x8 nan8 = {hn, hn, hn, hn, hn, hn, hn, hn};
    for (int t = k0; has(t); ++t) {
      int b, p, n_parts;
      if (!entry_unit(a, static_cast<uint32_t>(scalar_load(items, item(t))), b, p, n_parts))
        continue;
      for (int idx = lane; idx < G * (D / 8); idx += kWave)
        store_rows<D>(a, g, b, p, n_parts, idx / (D / 8), (idx % (D / 8)) * 8, nan8, nan, nan);
    }
  };
  auto abandoned = [&]() {
    return __hip_atomic_load(w.abandon, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != 0;
  };
  // both wavefronts: write ring slots 0 .. count-1 to their global rows
  auto flush = [&](int count) {
    for (int j = wave; j < count; j += kDecodeWaves) {
      const int4 info = w.ring_info[j];  // request, partition, partitions, valid
      if (info.w == 0) continue;
      for (int idx = lane; idx < G * (D / 8); idx += kWave) {
        const int h = idx / (D / 8);
        const int d0 = (idx % (D / 8)) * 8;
        const f16x8 r = *reinterpret_cast<const f16x8*>(w.ring_o + (j * G + h) * D + d0);
        store_rows<D>(a, g, info.x, info.y, info.z, h, d0, r, w.ring_m[j * G + h],
                      w.ring_l[j * G + h]);
      }
    }
  };

  if (MULTI ? k_end <= 0 : !has(0)) return;
  Unit u = has(0) ? unit_at(item(0)) : no_unit();
  typedef TileRegs<D, FP8> TR;
  f16x8 qf[D / 32];
  typename TR::K kA[TR::NB * TR::NK], kB[TR::NB * TR::NK];
  typename TR::V vA[TR::NB * TR::NV], vB[TR::NB * TR::NV];
  if (has(0)) load_q<D>(a, g, u.b, lane, qf);
  if (u.cnt > 0) load_set<D, KEEP, FP8>(a, g, u, no_unit(), 0, true, lane, kA, vA);

  int stop_k0 = 0;  // set when the loop is left early: the window to mark bad
  for (int k = 0;; ++k) {
    const bool more = has(k + 1);
    const bool last = MULTI ? k + 1 == k_end : !more;
    const Unit nx = more ? unit_at(item(k + 1)) : no_unit();
    WaveState<D> st;
    run_unit<D, KEEP, FP8>(a, g, wave, lane, u, nx, qf, kA, vA, kB, vB, st);
    if (more) load_q<D>(a, g, nx.b, lane, qf);  // in flight during the epilogue

    const int buf = k % kMergeSlots;
    const int k0 = k - k % ring;  // first unit of the ring window not yet flushed
    // slot `buf` was last used by unit k - kMergeSlots: wait until it has
    // been merged.  The wait is bounded: past spin_limit rounds (or once the
    // other wavefront has given up) the rest of the deal is written as NaN
    // rather than left stale, and the wavefront ends.
    int spins = 0;
    bool give_up = false;
    while (__hip_atomic_load(&w.merged[buf], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) !=
           k / kMergeSlots) {
      if (++spins > a.spin_limit || abandoned()) {
        give_up = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (give_up) {
      stop_k0 = k0;
      break;
    }
    const MergeSlot<D> ms{w.m + buf * kDecodeWaves * 16, w.l + buf * kDecodeWaves * 16,
                          w.o + buf * slot_floats, &w.arrive[buf], &w.bad[buf]};
    const int rs = k % ring;  // this unit's result slot
    if (post_state<D>(ms, st, G, wave, lane, u.bad)) {
      if (u.ok) {
        merge_unit<D, FP8>(ms, G, u.L, lane, a.v_scale,
                           [&](int h, int d0, f16x8 r, float m, float l) {
          *reinterpret_cast<f16x8*>(w.ring_o + (rs * G + h) * D + d0) = r;
          if (d0 == 0) {
            w.ring_m[rs * G + h] = m;
            w.ring_l[rs * G + h] = l;
          }
        });
      }
      if (lane == 0) {
        w.ring_info[rs] = int4{u.b, u.p, u.n_parts, u.ok ? 1 : 0};
        w.arrive[buf] = 0;
        w.bad[buf] = 0;
        __hip_atomic_fetch_add(&w.merged[buf], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
    if (last || rs == ring - 1) {
      // every unit in the ring has been merged once both wavefronts get here
      // (a wavefront that gave up has ended, and the barrier waits only for
      // the other one, which then writes the window as NaN instead)
      __syncthreads();
      if (abandoned()) {
        stop_k0 = k0;
        break;
      }
      flush(rs + 1);
      if (last) return;
      __syncthreads();  // the ring is read out before the next unit reuses slot 0
    }
    u = nx;
  }
  abandon(stop_k0);
}

// Work-list form: gridDim.y resident workgroups of one wavefront pair each
// per kv head; workgroup (g, y) is pair y of kv head g's walk.
template <int D, bool KEEP, bool FP8>
__global__ __launch_bounds__(kDecodeThreads) __attribute__((amdgpu_waves_per_eu(PA_WL_WAVES_PER_EU)))
void decode_worklist_kernel(DecodeArgs a, const int32_t* __restrict__ items, int32_t n_items,
                            int32_t ring) {
  __shared__ float sm_m[kMergeSlots * kDecodeWaves * 16];
  __shared__ float sm_l[kMergeSlots * kDecodeWaves * 16];
  __shared__ int sm_arrive[kMergeSlots];
  __shared__ int sm_bad[kMergeSlots];
  __shared__ int sm_merged[kMergeSlots];
  __shared__ int sm_abandon;
  // dynamic LDS: the merge rows, then the result ring
  extern __shared__ f32x4 sm_o4[];
  if (threadIdx.x < kMergeSlots) {
    sm_arrive[threadIdx.x] = 0;
    sm_bad[threadIdx.x] = 0;
    sm_merged[threadIdx.x] = 0;
  }
  if (threadIdx.x == 0) sm_abandon = 0;
  __syncthreads();
  const int G = a.G;
  WalkLds w;
  w.m = sm_m;
  w.l = sm_l;
  w.arrive = sm_arrive;
  w.bad = sm_bad;
  w.merged = sm_merged;
  w.abandon = &sm_abandon;
  w.o = reinterpret_cast<float*>(sm_o4);
  w.ring_info = reinterpret_cast<int4*>(w.o + kMergeSlots * kDecodeWaves * G * (D + 4));
  w.ring_o = reinterpret_cast<f16*>(w.ring_info + ring);
  w.ring_m = reinterpret_cast<float*>(w.ring_o + ring * G * D);
  w.ring_l = w.ring_m + ring * G;
  worklist_walk<D, KEEP, FP8, false>(a, items, n_items, ring, blockIdx.x, blockIdx.y,
                                     gridDim.y, 0, uniform(threadIdx.x >> 6), threadIdx.x & 63,
                                     w);
}

// Both pool types: pools, geometry and (FP8) scales, then the shared checks
// and launches.
struct PoolArgs {
  const void* k_pool;
  const void* v_pool;
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  bool fp8;
  float k_scale;
  float v_scale;
};

// Bound on the work-list kernel's LDS slot wait: kSpinLimit rounds, or the
// value of the environment variable PA_DECODE_SPIN_LIMIT (>= 0), a test hook
// that makes the give-up path run without anything hanging.
inline int32_t decode_spin_limit() {
  const char* e = getenv("PA_DECODE_SPIN_LIMIT");
  if (e == nullptr || *e == 0) return kSpinLimit;
  char* end = nullptr;
  const long v = strtol(e, &end, 10);
  return (end != e && v >= 0 && v <= kSpinLimit) ? static_cast<int32_t>(v) : kSpinLimit;
}

// Host checks of a decode batch's arguments, then its kernel arguments.  PA_OK
// with batch == 0 means there is nothing to launch.
static pa_status decode_prepare(pa_half* out, const pa_half* q, const PoolArgs& kv,
                                const int32_t* tables, int32_t max_blocks,
                                const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                                float scale, int32_t partition_size, int32_t max_seq_len,
                                const int32_t* work_items, int32_t n_items, void* workspace,
                                uint64_t workspace_bytes, uint32_t flags, DecodeArgs& a) {
  if (kv.k_pool == nullptr || kv.v_pool == nullptr || kv.block_size != kBlock ||
      kv.num_blocks <= 0 || kv.num_kv_heads <= 0 || kv.num_kv_heads > 65535)
    return PA_ERR_INVALID;
  if (kv.head_dim != 64 && kv.head_dim != 128) return PA_ERR_INVALID;
  if (batch < 0 || batch > 65535 || max_blocks < 0 || max_seq_len < 0) return PA_ERR_INVALID;
  if (num_q_heads <= 0 || num_q_heads % kv.num_kv_heads != 0) return PA_ERR_INVALID;
  const int G = num_q_heads / kv.num_kv_heads;
  if (G > 16) return PA_ERR_INVALID;
  if (partition_size <= 0 || partition_size % kBlock != 0 ||
      partition_size > kDecodeWaves * kMaxWaveBlocks * kBlock)
    return PA_ERR_INVALID;
  if (!scale_ok(scale)) return PA_ERR_INVALID;
  if (kv.fp8 && !(kv.k_scale > 0.0f && kv.k_scale <= 3.0e38f && kv.v_scale > 0.0f &&
                  kv.v_scale <= 3.0e38f))
    return PA_ERR_INVALID;
  if ((flags & ~static_cast<uint32_t>(PA_DECODE_KEEP_KV)) != 0) return PA_ERR_INVALID;
  if (n_items < 0 || n_items > (1 << 30) || (n_items > 0 && work_items == nullptr))
    return PA_ERR_INVALID;
  if (batch == 0) return PA_OK;
  if (out == nullptr || q == nullptr || tables == nullptr || seq_lens == nullptr ||
      !aligned16(q) || !aligned16(out) || !aligned16(kv.k_pool) || !aligned16(kv.v_pool))
    return PA_ERR_INVALID;
  if (static_cast<int64_t>(max_seq_len) > static_cast<int64_t>(max_blocks) * kBlock)
    return PA_ERR_INVALID;
  const int part_blocks = partition_size / kBlock;
  const int p_max = max_seq_len == 0 ? 1 : (max_seq_len + partition_size - 1) / partition_size;
  if (p_max > 65535) return PA_ERR_INVALID;
  const int D = kv.head_dim;
  const uint64_t need =
      pa_decode_workspace_bytes(batch, num_q_heads, D, max_seq_len, partition_size);
  if (p_max > 1 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)))
    return PA_ERR_INVALID;

  a.q = reinterpret_cast<const f16*>(q);
  a.kp = static_cast<const f16*>(kv.k_pool);
  a.vp = static_cast<const f16*>(kv.v_pool);
  a.tables = tables;
  a.seq_lens = seq_lens;
  a.batch = batch;
  a.spin_limit = decode_spin_limit();
  a.max_blocks = max_blocks;
  a.num_blocks = kv.num_blocks;
  a.n_kv = kv.num_kv_heads;
  a.G = G;
  // FP8: a score is scale * q . (code * k_scale); k_scale joins the exponent's factor
  a.scale_log2 = kv.fp8 ? scale * kv.k_scale * 1.4426950408889634f
                        : scale * 1.4426950408889634f;
  a.v_scale = kv.fp8 ? kv.v_scale : 1.0f;
  a.part_blocks = part_blocks;
  a.p_max = p_max;
  a.out = reinterpret_cast<f16*>(out);
  a.ws_o = nullptr;
  a.ws_m = nullptr;
  a.ws_l = nullptr;
  if (p_max > 1) {
    const int64_t slots = static_cast<int64_t>(batch) * num_q_heads * p_max;
    a.ws_o = static_cast<f16*>(workspace);
    a.ws_m = reinterpret_cast<float*>(a.ws_o + slots * D);
    a.ws_l = a.ws_m + slots;
  }
  return PA_OK;
}

}  // namespace pa
