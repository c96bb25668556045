// Paged-attention decode for gfx950: one query row per (sequence, query
// head) against the sequence's whole history, read block by block through
// its block table, with an online (running max / running sum) softmax
// (JuliaPagedAttn README, "Online Softmax" and "API Reference":
// paged_attention_cpu!; nanoserve Day 19, "What I added today": attend over
// the whole history through the block table in place).
//
// Work decomposition
//   A persistent grid of workgroups (eight waves, one workgroup per CU; four
//   for the register-heavy variants) walks segments of (sequence, KV head)
//   pairs: whole pairs, or, when the context is split, an equal static slice
//   of the batch's work per workgroup and then chunks handed out as the
//   workgroups finish (see the driver below); the waves of a workgroup take
//   a segment's blocks round-robin.
//   Inside a wave the 64 lanes form four 16-lane DPP rows.  Row r handles
//   tokens r, r+4, r+8, r+12 of the wave's current 16-token block; lane i of
//   the row owns elements [i*D/16, (i+1)*D/16) of the head dimension, so one
//   token row of one KV head (D elements) is read by 16 lanes with one
//   contiguous load each (16 bytes for bf16 at D = 128).
//   All n_rep query heads that share the KV head (GQA, nanoserve Day 19
//   "What I learned" item 4) are kept in every lane, so each K/V byte is
//   read once for the whole group.
//
// Scores: each lane forms n_rep partial dot products over its elements
// (v_dot2_f32_bf16 for bf16).  A DPP reduce-scatter across the row leaves
// every lane with the complete score of ONE head of the group: at each level
// a lane keeps half of its partial sums and adds its partner's other half
// (partners are the row mirror, the half-row mirror and two quad
// permutations, so no LDS traffic).  The query heads are loaded in a
// lane-dependent order that makes the halves line up.
//
// Softmax: each lane keeps the running max m and sum l of its own head and
// row (one independent token stream per row), in the log2 domain.  The
// probabilities and the rescale factor of all heads are broadcast back
// along the row with DPP rotations for the P.V accumulation, which is fp32.
//
// End of a segment: rows and then waves are merged with the same max/sum
// rescaling; a whole pair is normalised and written to `out`, a piece of a
// pair writes its (o/l, m, l) to the workspace, and the workgroup that
// counts the last piece of the pair combines them by log-sum-exp weights (an
// arrival counter per pair, no second kernel).

#include <float.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

// Waves per workgroup.  One workgroup of eight waves per CU streams a
// segment's blocks with all of them: the waves of one CU then share each
// segment instead of two workgroups of four competing for it (the older of
// two co-resident workgroups wins the issue arbitration and the younger one
// trails it by about a quarter).  Variants whose registers do not fit two
// waves per SIMD (wide fp32 rows with many query heads) keep four.
template <typename T, int D, int R>
constexpr int decode_waves() {
  constexpr int NW = D * static_cast<int>(sizeof(T)) / 64;       // dwords per lane per token row
  constexpr int footprint = 16 * NW + (1 << R) * (D / 16 + NW);  // ring + accumulators + query
  return footprint >= 160 ? 4 : 8;
}
constexpr float kNegBig = -1.0e30f;  // "no score yet": finite, so m - m stays 0
constexpr int kRing = 2;                    // blocks per wave in the load ring
constexpr float kRescaleLog2 = 8.f;         // reference-max slack before a rescale
constexpr int kKVPolicy = 2;                // K/V loads are non-temporal: each byte is read once

// Head index, relative to the lane's own head, held at position idx of the
// reduce-scatter input when the group has 2^R heads.  Level k of the scatter
// pairs lanes that differ in bit 3-k and every lower bit; the lane keeps
// the first half of its values, so position idx carries the XOR of the
// partner masks of the levels whose bit is set in idx.
template <int R>
__device__ __forceinline__ constexpr int scatter_head_xor(int idx) {
  int x = 0;
  for (int k = 0; k < R; ++k)
    if (idx & (1 << (R - 1 - k))) x ^= (1 << (R - k)) - 1;
  return x;
}

template <int K>
__device__ __forceinline__ float level_partner(float x) {
  if constexpr (K == 0) return dpp_mov<dpp::kRowMirror>(x);
  else if constexpr (K == 1) return dpp_mov<dpp::kRowHalfMirror>(x);
  else if constexpr (K == 2) return dpp_mov<dpp::kQuadReverse>(x);
  else return dpp_mov<dpp::kQuadSwapPairs>(x);
}

template <int R, int K>
__device__ __forceinline__ void scatter_level(float (&v)[1 << R]) {
  if constexpr (K < R) {
    constexpr int half = (1 << R) >> (K + 1);
#pragma unroll
    for (int j = 0; j < half; ++j) v[j] += level_partner<K>(v[j + half]);
  } else {
    v[0] += level_partner<K>(v[0]);
  }
}

// Sum over the 16 lanes of a row, scattered: returns the full score of the
// lane's own head (lane bits 3..4-R name the head).
template <int R>
__device__ __forceinline__ float reduce_scatter(float (&v)[1 << R]) {
  scatter_level<R, 0>(v);
  scatter_level<R, 1>(v);
  scatter_level<R, 2>(v);
  scatter_level<R, 3>(v);
  return v[0];
}

// Value of slot J along the row: slot 0 is the lane's own head, slot J>0
// comes from the lane J*W places away (W = 16 / heads).
template <int R, int J>
__device__ __forceinline__ float row_bcast(float x) {
  if constexpr (J == 0) return x;
  else return dpp_mov<dpp::row_ror(J * (16 >> R))>(x);
}
template <int R, int J>
__device__ __forceinline__ int row_bcast_i(int x) {
  if constexpr (J == 0) return x;
  else return dpp_mov_i<dpp::row_ror(J * (16 >> R))>(x);
}

template <int R, int J = 0>
__device__ __forceinline__ void bcast_all(float x, float (&dst)[1 << R]) {
  if constexpr (J < (1 << R)) {
    dst[J] = row_bcast<R, J>(x);
    bcast_all<R, J + 1>(x, dst);
  }
}
template <int R, int J = 0>
__device__ __forceinline__ void bcast_all_i(int x, int (&dst)[1 << R]) {
  if constexpr (J < (1 << R)) {
    dst[J] = row_bcast_i<R, J>(x);
    bcast_all_i<R, J + 1>(x, dst);
  }
}

// Element traits: T is the storage type (float or uint16_t for bf16).
template <typename T, int D>
struct Layout {
  static constexpr int kElt = sizeof(T);
  static constexpr int kEPL = D / 16;                // elements per lane
  static constexpr int kNW = kEPL * kElt / 4;        // dwords per lane per token row
};

template <typename T, int D>
__device__ __forceinline__ float frag_dot(const uint32_t (&q)[Layout<T, D>::kNW],
                                          const Frag<Layout<T, D>::kNW>& k, float acc) {
  constexpr int NW = Layout<T, D>::kNW;
  if constexpr (sizeof(T) == 2) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int w = 0; w < NW; ++w)
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q[w]),
                                            __builtin_bit_cast(bf16x2, k.w[w]), acc, false);
  } else {
#pragma unroll
    for (int w = 0; w < NW; ++w) acc = fmaf(__uint_as_float(q[w]), __uint_as_float(k.w[w]), acc);
  }
  return acc;
}

template <typename T, int D>
__device__ __forceinline__ float frag_elem(const Frag<Layout<T, D>::kNW>& f, int e) {
  if constexpr (sizeof(T) == 2) return (e & 1) ? bf16_hi(f.w[e >> 1]) : bf16_lo(f.w[e >> 1]);
  else return __uint_as_float(f.w[e]);
}

template <typename T>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float v) {
  if constexpr (sizeof(T) == 2) static_cast<uint16_t*>(out)[idx] = f32_to_bf16(v);
  else static_cast<float*>(out)[idx] = v;
}

// Partition results travel between workgroups that may sit on different
// dies: device-scope (agent) atomic stores and loads, which on gfx950 are
// issued at the device-coherent level (sc1: written through, and read past,
// a die's own L2).  Their order is set by the pair's arrival counter (see
// the arrivals at the end of the kernel).
__device__ __forceinline__ void store_shared(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_shared(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Log-sum-exp merge of the pieces of one (sequence, KV head) pair, for the
// N query heads of its group: out = sum_j w_j o_j / sum_j w_j with
// w_j = l_j * 2^(m_j - max m), o_j a piece's normalised output (JuliaPagedAttn
// "Online Softmax": the same max/sum rescaling that joins two blocks joins
// two pieces), taken in token order with a running maximum.  The pair's
// blocks sit at work positions [A, E) and its work range starts at A0 <= A;
// its piece in unit i (a static slice or a chunk, numbered in position order)
// sits in partial slot 2i, or 2i + 1 for the first unit when that unit starts
// before the pair's work range (then an earlier pair's segment came first in
// it).  Each thread owns E_
// output elements; the loads of eight pieces are issued together, so a merge
// of up to eight pieces costs one memory round trip.
constexpr int kMergeBatch = 8;

template <typename T, int D, int N, int kThreads>
__device__ __forceinline__ void merge_pair(const DecodeArgs& a, int s, int g, int A0, int A,
                                           int E, const UnitPlan& up, int tid) {
  constexpr int kOut = N * D;
  constexpr int E_ = (kOut + kThreads - 1) / kThreads;
  const int ia = up.of(A);
  const int n = up.of(E - 1) - ia + 1;
  const bool first_tail = up.start(ia) < A0;
  float M[E_], wsum[E_], osum[E_];
  int hd[E_], dd[E_];
#pragma unroll
  for (int e = 0; e < E_; ++e) {
    const int o = min(tid + e * kThreads, kOut - 1);
    hd[e] = o / D;
    dd[e] = o - hd[e] * D;
    M[e] = kNegBig;
    wsum[e] = 0.f;
    osum[e] = 0.f;
  }
  for (int j0 = 0; j0 < n; j0 += kMergeBatch) {
    float mj[E_][kMergeBatch], lj[E_][kMergeBatch], oj[E_][kMergeBatch];
#pragma unroll
    for (int jj = 0; jj < kMergeBatch; ++jj) {
      const int i = ia + min(j0 + jj, n - 1);   // past the end: reload the last, weight 0
      const int slot = (i == ia && first_tail) ? 2 * i + 1 : 2 * i;
#pragma unroll
      for (int e = 0; e < E_; ++e) {
        const int64_t r = static_cast<int64_t>(slot) * N + hd[e];
        mj[e][jj] = load_shared(a.part_ml + r * 2);
        lj[e][jj] = load_shared(a.part_ml + r * 2 + 1);
        oj[e][jj] = load_shared(a.part_o + r * D + dd[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < E_; ++e)
#pragma unroll
      for (int jj = 0; jj < kMergeBatch; ++jj) {
        if (j0 + jj >= n) break;
        if (mj[e][jj] > M[e]) {
          const float c = fast_exp2(M[e] - mj[e][jj]);
          wsum[e] *= c;
          osum[e] *= c;
          M[e] = mj[e][jj];
        }
        const float w = lj[e][jj] * fast_exp2(mj[e][jj] - M[e]);
        wsum[e] += w;
        osum[e] = fmaf(w, oj[e][jj], osum[e]);
      }
  }
  const int64_t row0 = static_cast<int64_t>(s) * a.num_q_heads + g * N;
#pragma unroll
  for (int e = 0; e < E_; ++e) {
    const int o = tid + e * kThreads;
    if (o < kOut)
      store_out<T>(a.out, row0 * D + o, osum[e] * (wsum[e] > 0.f ? 1.f / wsum[e] : 0.f));
  }
}

// Persistent driver.  Each workgroup first builds, in LDS, the plan of the
// whole batch: clamped context lengths and the prefix sum of the work per KV
// head.  Pair p = s * Hkv + g (sequence s, KV head g) owns nb_s =
// ceil(L_s / 16) blocks.  Its work is priced at c_s = nb_s + seg_cost
// block-equivalents (0 for an empty context): the blocks, plus the fixed
// cost of a segment (its epilogue and the restart of its load ring), so
// that a slice full of short pairs is not overloaded.  The pairs' work
// ranges lie end to end at W_p = Hkv * pre_s + g * c_s, B in all; block j
// of the pair sits at W_p + seg_cost + j.
//
// Split (min_slice_blocks > 0): the work range is cut into units (unit_plan):
// one static slice per workgroup, workgroup i taking slice i, so every
// workgroup gets the same work whatever the mix of context lengths; when the
// non-empty pairs differ in length the slices cover nine tenths of it and
// the rest is cut into chunks that the workgroups take from a counter as
// they finish, so the ones that run slower (their speed differs by die and
// by CU, from call to call alike) take fewer.  The part of a pair inside a
// unit (a segment: the pair's blocks whose positions fall in the unit) keeps
// its own online-softmax state.  Only the first and the last segment of a
// unit can be pieces of a pair that goes on in another unit; they write
// (o, m, l) to partial slots 2u and 2u + 1, the segments between them are
// whole pairs and write `out`.  At the end of a unit its workgroup counts
// its pieces at their pairs' arrival counters, and the last arrival of a
// pair merges it.  Which workgroup computes a unit does not change what it
// computes, so the result is the same bit for bit from call to call.
// Without a split, workgroup i takes pairs i, i + grid, ... whole.
//
// Inside a segment the waves take its blocks round-robin, each through
// a ring of kRing register buffers (kRing-1 blocks in flight while one is
// computed).  Between segments nothing drains: while one computes, the table
// entries of the next are already loaded, and the query rows and first ring
// blocks of the next are issued right after the output stores, so the memory
// pipe stays busy across boundaries.  Every wait the compiler places inside
// the ring is then exact, because whatever reaches the ring's loop header has
// the primed blocks as its youngest loads.
//
// Plan in dynamic LDS: ctx[S] clamped context lengths, pre[S+1] exclusive
// prefix sum of blocks per KV head.
//
// kStep: the decode step in one launch (pa_decode_step).  Each sequence's
// new token (position context_lens[s] - 1) is written to its slot by one
// workgroup, exactly as pa_append_kv writes it, and its slot recorded.
// The wave whose 16-token unit holds that position does not read the row
// back from the pool: its loads of that row are pointed past their
// descriptor (no memory access) and the row's fragments come from k_new and
// v_new instead, loaded when the segment starts.  No location is then both
// written and read in one call, and the result equals pa_append_kv followed
// by pa_decode bit for bit.
template <typename T, int D, int R, bool kSmall, bool kStep>
__global__ __launch_bounds__((64 * decode_waves<T, D, R>())) void decode_kernel(DecodeArgs a) {
  constexpr int kWaves = decode_waves<T, D, R>();
  constexpr int kThreads = 64 * kWaves;
  constexpr int kChunkBlocks = 64 * kWaves;  // blocks whose table entries one load brings in
  using LT = Layout<T, D>;
  constexpr int N = 1 << R;          // query heads per KV head
  constexpr int W = 16 >> R;         // lanes per head after the reduce-scatter
  constexpr int EPL = LT::kEPL;
  constexpr int NW = LT::kNW;
  using F = Frag<NW>;

  extern __shared__ int32_t sm_plan[];
  __shared__ int32_t sm_scan[kThreads];
  __shared__ float sm_acc[kWaves][N][D];
  __shared__ float sm_m[kWaves][N];
  __shared__ float sm_l[kWaves][N];
  __shared__ int sm_last[2];
  __shared__ int sm_nb[kWaves][2];   // per wave: least and most blocks of a non-empty pair
  __shared__ int sm_unit;
  // kStep: 1 where the sequence's new token lies inside its clamped context
  __shared__ uint8_t sm_new[kStep ? kMaxDecodeSeqs : 1];

  const int S = a.num_seqs;
  const int Hkv = a.num_kv_heads;
  int32_t* const sm_ctx = sm_plan;
  int32_t* const sm_pre = sm_plan + S;
  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63;
  const int row = lane >> 4;
  const int li = lane & 15;

  // ---- the plan --------------------------------------------------------------
  {
    const int per = (S + kThreads - 1) / kThreads;   // run of sequences per thread
    const int b0 = min(S, tid * per);
    const int b1 = min(S, b0 + per);
    int cb = 0;
    int nb_lo = 0x7fffffff, nb_hi = 0;
    for (int q = b0; q < b1; ++q) {
      int L = a.context_lens[q];
      if constexpr (kStep) sm_new[q] = L >= 1 && L <= a.context_cap;
      L = L < 0 ? 0 : (L > a.context_cap ? a.context_cap : L);
      sm_ctx[q] = L;
      const int nbq = (L + kUnit - 1) / kUnit;
      cb += L > 0 ? nbq + a.seg_cost : 0;
      if (L > 0) {
        nb_lo = min(nb_lo, nbq);
        nb_hi = max(nb_hi, nbq);
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      nb_lo = min(nb_lo, __shfl_xor(nb_lo, off));
      nb_hi = max(nb_hi, __shfl_xor(nb_hi, off));
    }
    if (lane == 0) {
      sm_nb[wave][0] = nb_lo;
      sm_nb[wave][1] = nb_hi;
    }
    sm_scan[tid] = cb;
    __syncthreads();
    if (tid < 64) {
      // exclusive scan of the per-thread counts: kThreads / 64 per lane, then the wave
      int c[kThreads / 64], t = 0;
#pragma unroll
      for (int i = 0; i < kThreads / 64; ++i) {
        c[i] = sm_scan[kThreads / 64 * tid + i];
        t += c[i];
      }
      int x = t;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (tid >= off) x += y;
      }
      int e = x - t;
#pragma unroll
      for (int i = 0; i < kThreads / 64; ++i) {
        sm_scan[kThreads / 64 * tid + i] = e;
        e += c[i];
      }
      if (tid == 63) sm_pre[S] = x;
    }
    __syncthreads();
    int e = sm_scan[tid];
    for (int q = b0; q < b1; ++q) {
      sm_pre[q] = e;
      e += sm_ctx[q] > 0 ? (sm_ctx[q] + kUnit - 1) / kUnit + a.seg_cost : 0;
    }
    __syncthreads();
  }
  // an empty context gives zeros: its sequence's rows, spread over the grid
  for (int q = blockIdx.x; q < S; q += gridDim.x) {
    if (sm_ctx[q] == 0) {
      for (int o = tid; o < a.num_q_heads * D; o += kThreads)
        store_out<T>(a.out, static_cast<int64_t>(q) * a.num_q_heads * D + o, 0.f);
    }
  }

  // ---- segments ---------------------------------------------------------------
  const bool split = a.min_slice_blocks > 0;
  const int n_pairs = S * Hkv;
  const int B = Hkv * sm_pre[S];               // the host keeps this below 2^31
  UnitPlan up{};                               // split: static slices, then handed-out chunks
  if (split) {
    int nb_lo = 0x7fffffff, nb_hi = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      nb_lo = min(nb_lo, sm_nb[w][0]);
      nb_hi = max(nb_hi, sm_nb[w][1]);
    }
    up = unit_plan(B, static_cast<int>(gridDim.x), a.min_slice_blocks, a.max_slices,
                   nb_lo >= nb_hi);
  }
  int u = blockIdx.x;                          // split: the unit being walked
  int F0 = 0, F1 = 0;                          // its work range [F0, F1)
  const int C = a.seg_cost;
  auto nb_of = [&](int q) { return (sm_ctx[q] + kUnit - 1) / kUnit; };
  auto cost_of = [&](int q) { return sm_pre[q + 1] - sm_pre[q]; };
  struct Seg {
    int s, g, L, tok1, blk0, blk1;
    int slot;                        // partial slot, or -1: a whole pair, written to out
    int end;                         // split: work position just past the segment
  };
  // segment starting at `pos`: a flat block (split) or a pair index
  // segment of the pair whose work range holds `pos` (split: a work
  // position; may be empty when the slice ends before the pair's first block)
  auto seg_at = [&](int pos) {
    Seg x;
    if (split) {
      // last sequence whose work starts at or before pos (a run of empty
      // sequences ends at the one that owns the position)
      int lo = 0, hi = S - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (Hkv * sm_pre[mid] <= pos) lo = mid; else hi = mid - 1;
      }
      x.s = lo;
      const int nb = nb_of(lo);
      const int cw = cost_of(lo);
      const int off = pos - Hkv * sm_pre[lo];
      x.g = off / cw;
      const int first_blk = Hkv * sm_pre[lo] + x.g * cw + C;   // work position of block 0
      x.blk0 = max(0, pos - first_blk);
      x.blk1 = min(nb, F1 - first_blk);
      x.end = first_blk + x.blk1;
      x.slot = (x.blk0 == 0 && x.blk1 == nb) ? -1
             : 2 * u + (pos == F0 ? 0 : 1);
    } else {
      x.s = pos / Hkv;
      x.g = pos - x.s * Hkv;
      x.blk0 = 0;
      x.blk1 = nb_of(x.s);
      x.slot = -1;
    }
    x.L = sm_ctx[x.s];
    x.tok1 = min(x.blk1 * kUnit, x.L);
    return x;
  };
  auto skip_empty = [&](int p) {
    while (p < n_pairs && nb_of(p / Hkv) == 0) p += gridDim.x;
    return p;
  };
  auto next_pos = [&](const Seg& x, int pos) {
    return split ? x.end : skip_empty(pos + gridDim.x);
  };
  int pos_end = n_pairs;
  // lane t: table entries of this wave's t-th 16-token unit of the chunk at
  // c0.  Unit j holds positions 16 j .. 16 j + 15: with blocks of 16 tokens
  // or more, the rows 16 j mod B .. of block 16 j / B; with blocks of 8, two
  // blocks, 2 j and 2 j + 1 (.y; the same block as .x otherwise)
  const uint32_t bshift = a.geom.block_shift;
  constexpr bool small = kSmall;     // blocks of 8 tokens (block_shift 3)
  auto load_tbl = [&](const Seg& x, int c0) {
    const int j = c0 + wave + kWaves * lane;
    const int e = (j << 4) >> bshift;
    const int32_t* row = a.block_tables + static_cast<int64_t>(x.s) * a.max_blocks_per_seq;
    int2 t = make_int2(-1, -1);
    if (j < x.blk1) {
      t.x = e < a.max_blocks_per_seq ? row[e] : -1;
      if constexpr (small) t.y = e + 1 < a.max_blocks_per_seq ? row[e + 1] : -1;
    }
    return t;
  };
  const int own = li >> (4 - R);     // head whose full score this lane ends with
  // query rows of the segment's heads, in this lane's scatter order
  auto load_q = [&](const Seg& x, uint32_t (&qd)[N][NW]) {
    const char* qb = static_cast<const char*>(a.q) +
                     ((static_cast<int64_t>(x.s) * a.num_q_heads + x.g * N) * D + li * EPL) * LT::kElt;
#pragma unroll
    for (int idx = 0; idx < N; ++idx) {
      const int h = own ^ scatter_head_xor<R>(idx);
      const F f = load_frag<NW>(qb + static_cast<int64_t>(h) * D * LT::kElt);
#pragma unroll
      for (int w = 0; w < NW; ++w) qd[idx][w] = f.w[w];
    }
  };

  int slot_head[N];                  // head carried by accumulator slot j
  bcast_all_i<R>(own, slot_head);

  // token rows of one KV head: token_stride apart, head_stride between heads
  // (token-major or head-major blocks); a block's rows fill `span` bytes
  const uint32_t row_bytes = a.geom.token_stride;
  const uint32_t head_bytes = a.geom.head_stride;
  const uint32_t block_bytes = a.geom.span;
  const int64_t block_stride = a.geom.block_stride;
  const char* kpool = static_cast<const char*>(a.k_cache);
  const char* vpool = static_cast<const char*>(a.v_cache);
  const float sl2 = a.scale_log2;

  // ---- units: the slice of this workgroup, then chunks handed out (split);
  // without a split, the workgroup's whole pairs --------------------------------
  int* const ctl = a.counters + kPairSlots;   // [0] units handed out, [1] workgroups done
  for (;;) {
    if (split) {
      F0 = up.start(u);
      F1 = up.end(u);
      pos_end = F1;
    }
    // pieces of pairs stored by this unit: its first segment (slot 2u) and its
    // last (slot 2u + 1), counted at its end
    int pa_s = -1, pa_g = 0, pb_s = -1, pb_g = 0;
    int pos = split ? F0 : skip_empty(blockIdx.x);
    Seg cur;
    bool any = pos < pos_end;
    if (any) {
      cur = seg_at(pos);
      any = cur.blk1 > cur.blk0;     // else the unit holds no block
    }
    if (any) {
      int c0 = cur.blk0;                 // first block of the current chunk
      int nk = 0;                        // this wave's blocks in the current chunk
      int2 tbl = load_tbl(cur, c0);
      uint32_t qv[N][NW];
      load_q(cur, qv);
      // kStep: the unit of the segment that holds its pair's new token (-1:
      // none), the token's row in that unit, and the row's fragments
      int newj = -1, newt = 0;
      F knew, vnew;
      auto step_row = [&](const Seg& x) {
        newj = -1;
        if constexpr (kStep) {
          const int jn = (x.L - 1) >> 4;
          if (sm_new[x.s] && jn >= x.blk0 && jn < x.blk1) {
            newj = jn;
            newt = (x.L - 1) & 15;
            const int64_t o = ((static_cast<int64_t>(x.s) * Hkv + x.g) * D + li * EPL) * LT::kElt;
            knew = load_frag<NW>(static_cast<const char*>(a.k_new) + o);
            vnew = load_frag<NW>(static_cast<const char*>(a.v_new) + o);
          }
        }
      };
      step_row(cur);
      uint32_t lane_off = cur.g * head_bytes + li * EPL * LT::kElt + row * row_bytes;
      auto chunk_blocks = [&](const Seg& x, int cs) {
        const int ce = min(x.blk1, cs + kChunkBlocks);
        return ce - cs - wave > 0 ? (ce - cs - wave + kWaves - 1) / kWaves : 0;
      };

      float m = kNegBig, l = 0.f;
      float acc[N][EPL];
    #pragma unroll
      for (int j = 0; j < N; ++j)
    #pragma unroll
        for (int e = 0; e < EPL; ++e) acc[j][e] = 0.f;

      // Issue the loads of this wave's k-th unit of the current chunk into
      // (kf, vf) and return the mask of its valid tokens (bit t: token 16 j + t).
      // Past the wave's last unit, or for a table entry outside the pool, the
      // descriptors have size 0: the loads return zeros without touching memory
      // and the tokens of that block count as invalid.  Token rows 0 .. 7 of the
      // unit (uu = 0, 1) come through the first descriptor, rows 8 .. 15 through
      // the second, which is the first one again unless blocks hold 8 tokens.
      auto issue = [&](int k, F (&kf)[4], F (&vf)[4]) {
        int phys = -1, phys2 = -1;
        int nvalid = 0;
        int sub = 0;                     // first token row of the unit inside its block
        bool has_new = false;            // kStep: the unit holds the pair's new token
        if (k < nk) {
          const int j = c0 + wave + kWaves * k;
          if constexpr (kStep) has_new = j == newj;
          phys = __builtin_amdgcn_readlane(tbl.x, k);
          phys2 = small ? __builtin_amdgcn_readlane(tbl.y, k) : phys;
          const int n = cur.tok1 - j * kUnit;
          nvalid = n < kUnit ? n : kUnit;
          sub = small ? 0 : (j << 4) & ((1 << bshift) - 1);
        }
        const bool ok = phys >= 0 && phys < a.num_blocks;
        const bool ok2 = phys2 >= 0 && phys2 < a.num_blocks;
        const int vmask = ((ok ? 0x00ff : 0) | (ok2 ? 0xff00 : 0)) & ((1 << nvalid) - 1);
        const uint32_t sub_bytes = static_cast<uint32_t>(sub) * row_bytes;
        const int64_t off = ok ? static_cast<int64_t>(phys) * block_stride + sub_bytes : 0;
        const uint32_t size = ok ? block_bytes - sub_bytes : 0u;
        const Rsrc rk = make_rsrc(kpool + off, size);
        const Rsrc rv = make_rsrc(vpool + off, size);
        const int64_t off2 = ok2 ? static_cast<int64_t>(phys2) * block_stride : 0;
        const Rsrc rk2 = small ? make_rsrc(kpool + off2, ok2 ? block_bytes : 0u) : rk;
        const Rsrc rv2 = small ? make_rsrc(vpool + off2, ok2 ? block_bytes : 0u) : rv;
        const uint32_t lane_off2 = small ? lane_off - 8 * row_bytes : lane_off;
        uint32_t offs[4];
    #pragma unroll
        for (int uu = 0; uu < 4; ++uu) offs[uu] = (uu < 2 ? lane_off : lane_off2) + uu * 4 * row_bytes;
        if constexpr (kStep) {
          // the new token's row (lanes of row newt mod 4, fragment newt / 4) is
          // not read: an offset at the descriptor's size loads zeros, touching
          // nothing
          if (has_new && row == (newt & 3)) {
            const uint32_t past2 = small ? (ok2 ? block_bytes : 0u) : size;
    #pragma unroll
            for (int uu = 0; uu < 4; ++uu)
              if (uu == (newt >> 2)) offs[uu] = uu < 2 ? size : past2;
          }
        }
    #pragma unroll
        for (int uu = 0; uu < 2; ++uu)
          kf[uu] = load_frag_buf<NW, kKVPolicy>(rk, offs[uu]);
    #pragma unroll
        for (int uu = 2; uu < 4; ++uu)
          kf[uu] = load_frag_buf<NW, kKVPolicy>(rk2, offs[uu]);
    #pragma unroll
        for (int uu = 0; uu < 2; ++uu)
          vf[uu] = load_frag_buf<NW, kKVPolicy>(rv, offs[uu]);
    #pragma unroll
        for (int uu = 2; uu < 4; ++uu)
          vf[uu] = load_frag_buf<NW, kKVPolicy>(rv2, offs[uu]);
        return has_new ? (vmask | 0x10000) : vmask;
      };

      // Online softmax over one block (JuliaPagedAttn "Online Softmax"): scores,
      // running max and sum, then P.V.  The reference max of a stream only moves
      // when a score passes it by more than kRescaleLog2 (then the accumulators
      // are rescaled); in between, weights exp2(z - m) may exceed 1 (up to
      // 2^kRescaleLog2), which leaves sum(w v) / sum(w) unchanged.
      auto process = [&](F (&kf)[4], F (&vf)[4], int vmask) {
        if constexpr (kStep) {
          // the unit holding the new token: its row from k_new / v_new
          if (vmask & 0x10000) {
    #pragma unroll
            for (int uu = 0; uu < 4; ++uu) {
              if (uu == (newt >> 2) && row == (newt & 3)) {
                kf[uu] = knew;
                vf[uu] = vnew;
              }
            }
          }
          vmask &= 0xffff;
        }
        float z[4];
    #pragma unroll
        for (int uu = 0; uu < 4; ++uu) {
          float part_dot[N];
    #pragma unroll
          for (int idx = 0; idx < N; ++idx) part_dot[idx] = frag_dot<T, D>(qv[idx], kf[uu], 0.f);
          z[uu] = reduce_scatter<R>(part_dot) * sl2;
        }
        // tokens past the context (partial last unit, or a unit the ring runs
        // past its end) or in a block outside the pool get no weight and a zero
        // value row, whatever the pool holds there
        if (vmask != 0xffff) {
    #pragma unroll
          for (int uu = 0; uu < 4; ++uu) {
            if (((vmask >> (row + 4 * uu)) & 1) == 0) {
              z[uu] = -INFINITY;
    #pragma unroll
              for (int w = 0; w < NW; ++w) vf[uu].w[w] = 0u;
            }
          }
        }
        const float mx = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
        if (__builtin_amdgcn_ballot_w64(mx > m + kRescaleLog2) != 0) {
          const float m_new = mx > m + kRescaleLog2 ? mx : m;
          const float alpha = fast_exp2(m - m_new);
          m = m_new;
          l *= alpha;
          float alpha_j[N];
          bcast_all<R>(alpha, alpha_j);
    #pragma unroll
          for (int j = 0; j < N; ++j)
    #pragma unroll
            for (int e = 0; e < EPL; ++e) acc[j][e] *= alpha_j[j];
        }
        float p[4];
    #pragma unroll
        for (int uu = 0; uu < 4; ++uu) p[uu] = fast_exp2(z[uu] - m);

        if constexpr (sizeof(T) == 2) {
          // bf16: acc += p_a v_a + p_b v_b for token pairs (a, b) = (0, 1), (2, 3)
          // with one v_dot2_f32_bf16 per (head, element): the value rows of the
          // pair are interleaved with v_perm, the weights packed to bf16.  The
          // running sum adds the same rounded weights (slot 0 is the lane's own
          // head), so the normalised output is a convex combination of the V rows.
          typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
          typedef float f32x2 __attribute__((ext_vector_type(2)));
    #pragma unroll
          for (int pr = 0; pr < 2; ++pr) {
            const int ua = 2 * pr, ub = 2 * pr + 1;
            float pa[N], pb[N];
            bcast_all<R>(p[ua], pa);
            bcast_all<R>(p[ub], pb);
            uint32_t pw[N];
    #pragma unroll
            for (int j = 0; j < N; ++j) {
              const f32x2 two = {pa[j], pb[j]};
              pw[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(two, bf16x2));
            }
            l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[0]),
                                                __builtin_bit_cast(bf16x2, 0x3f803f80u), l, false);
    #pragma unroll
            for (int w = 0; w < NW; ++w) {
              // element 2w: low halves of token a and b; element 2w+1: high halves
              const uint32_t ve = __builtin_amdgcn_perm(vf[ub].w[w], vf[ua].w[w], 0x05040100u);
              const uint32_t vo = __builtin_amdgcn_perm(vf[ub].w[w], vf[ua].w[w], 0x07060302u);
    #pragma unroll
              for (int j = 0; j < N; ++j) {
                acc[j][2 * w] = __builtin_amdgcn_fdot2_f32_bf16(
                    __builtin_bit_cast(bf16x2, pw[j]), __builtin_bit_cast(bf16x2, ve), acc[j][2 * w],
                    false);
                acc[j][2 * w + 1] = __builtin_amdgcn_fdot2_f32_bf16(
                    __builtin_bit_cast(bf16x2, pw[j]), __builtin_bit_cast(bf16x2, vo),
                    acc[j][2 * w + 1], false);
              }
            }
          }
        } else {
          l += (p[0] + p[1]) + (p[2] + p[3]);
    #pragma unroll
          for (int uu = 0; uu < 4; ++uu) {
            float pj[N];
            bcast_all<R>(p[uu], pj);
    #pragma unroll
            for (int e = 0; e < EPL; ++e) {
              const float v = frag_elem<T, D>(vf[uu], e);
    #pragma unroll
              for (int j = 0; j < N; ++j) acc[j][e] = fmaf(pj[j], v, acc[j][e]);
            }
          }
        }
      };

      // ---- prologue: the first segment's table and query rows, then the next one's
      // (left in flight), then the first segment's primed ring blocks --------------
      __builtin_amdgcn_s_waitcnt(0);
      int pos_n = next_pos(cur, pos);
      bool has_next = pos_n < pos_end;
      Seg nxt = has_next ? seg_at(pos_n) : cur;
      has_next = has_next && nxt.blk1 > nxt.blk0;
      int2 tbl_nxt = has_next ? load_tbl(nxt, nxt.blk0) : make_int2(-1, -1);
      nk = chunk_blocks(cur, c0);

      F k0[4], v0[4], k1[4], v1[4], k2[4], v2[4];
      int n0 = issue(0, k0, v0);
      __builtin_amdgcn_sched_barrier(0);
      int n1 = 0;
      if constexpr (kRing == 3) n1 = issue(1, k1, v1);
      __builtin_amdgcn_sched_barrier(0);
      int n2 = 0;

      for (;;) {
        // ---- the ring over this chunk of the current segment (one exit, at the
        // bottom: a trip always runs every stage; stages past the wave's last
        // block see size-0 descriptors and zero valid tokens and change nothing)
        if constexpr (kRing == 2) {
          for (int k = 0; k < nk; k += 2) {
            n1 = issue(k + 1, k1, v1);
            __builtin_amdgcn_sched_barrier(0);
            process(k0, v0, n0);
            n0 = issue(k + 2, k0, v0);
            __builtin_amdgcn_sched_barrier(0);
            process(k1, v1, n1);
          }
        } else {
          for (int k = 0; k < nk; k += 3) {
            n2 = issue(k + 2, k2, v2);
            __builtin_amdgcn_sched_barrier(0);
            process(k0, v0, n0);
            n0 = issue(k + 3, k0, v0);
            __builtin_amdgcn_sched_barrier(0);
            process(k1, v1, n1);
            n1 = issue(k + 4, k1, v1);
            __builtin_amdgcn_sched_barrier(0);
            process(k2, v2, n2);
          }
        }

        // ---- a segment longer than one chunk: next chunk of the same segment -----
        if (c0 + kChunkBlocks < cur.blk1) {
          c0 += kChunkBlocks;
          tbl = load_tbl(cur, c0);
          __builtin_amdgcn_s_waitcnt(0);
          nk = chunk_blocks(cur, c0);
          n0 = issue(0, k0, v0);
          __builtin_amdgcn_sched_barrier(0);
          n1 = issue(1, k1, v1);
          __builtin_amdgcn_sched_barrier(0);
          continue;
        }

        // ---- merge the four rows of each wave -------------------------------------
        {
          float ms[N], ls[N];
          bcast_all<R>(m, ms);
          bcast_all<R>(l, ls);
    #pragma unroll
          for (int off = 16; off <= 32; off <<= 1) {
    #pragma unroll
            for (int j = 0; j < N; ++j) {
              const float mo = __shfl_xor(ms[j], off);
              const float lo = __shfl_xor(ls[j], off);
              const float mn = fmaxf(ms[j], mo);
              const float ca = fast_exp2(ms[j] - mn);
              const float cb = fast_exp2(mo - mn);
              ls[j] = ls[j] * ca + lo * cb;
              ms[j] = mn;
    #pragma unroll
              for (int e = 0; e < EPL; ++e)
                acc[j][e] = acc[j][e] * ca + __shfl_xor(acc[j][e], off) * cb;
            }
          }
          // ---- merge the waves through LDS ------------------------------------------
          if (row == 0) {
    #pragma unroll
            for (int j = 0; j < N; ++j)
    #pragma unroll
              for (int e = 0; e < EPL; ++e) sm_acc[wave][slot_head[j]][li * EPL + e] = acc[j][e];
            if ((li & (W - 1)) == 0) {
              sm_m[wave][own] = ms[0];
              sm_l[wave][own] = ls[0];
            }
          }
        }
        __syncthreads();
        {
          const bool direct = cur.slot < 0;
          for (int o = tid; o < N * D; o += kThreads) {
            const int h = o / D;
            const int d = o - h * D;
            float M = sm_m[0][h];
    #pragma unroll
            for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm_m[w][h]);
            float lsum = 0.f, osum = 0.f;
    #pragma unroll
            for (int w = 0; w < kWaves; ++w) {
              const float c = fast_exp2(sm_m[w][h] - M);
              lsum += sm_l[w][h] * c;
              osum += sm_acc[w][h][d] * c;
            }
            const float val = lsum > 0.f ? osum / lsum : 0.f;
            const int qh = cur.g * N + h;
            if (direct) {
              store_out<T>(a.out, (static_cast<int64_t>(cur.s) * a.num_q_heads + qh) * D + d, val);
            } else {
              const int64_t pi = static_cast<int64_t>(cur.slot) * N + h;
              store_shared(a.part_o + pi * D + d, val);
              if (d == 0) {
                store_shared(a.part_ml + pi * 2 + 0, M);
                store_shared(a.part_ml + pi * 2 + 1, lsum);
              }
            }
          }
        }
        __syncthreads();   // LDS merge buffers are reused by the next segment
        if (cur.slot >= 0) {
          if (cur.slot & 1) { pb_s = cur.s; pb_g = cur.g; }
          else { pa_s = cur.s; pa_g = cur.g; }
        }
        if (!has_next) break;

        // ---- move on: loads of the segment after next, then the next segment's
        // primed ring blocks (in that order, so the primed blocks are the
        // youngest loads)
        cur = nxt;
        pos = pos_n;
        pos_n = next_pos(cur, pos);
        has_next = pos_n < pos_end;
        if (has_next) {
          nxt = seg_at(pos_n);
          has_next = nxt.blk1 > nxt.blk0;
        }
        tbl = tbl_nxt;
        load_q(cur, qv);
        step_row(cur);
        tbl_nxt = has_next ? load_tbl(nxt, nxt.blk0) : make_int2(-1, -1);
        c0 = cur.blk0;
        nk = chunk_blocks(cur, c0);
        lane_off = cur.g * head_bytes + li * EPL * LT::kElt + row * row_bytes;
        m = kNegBig;
        l = 0.f;
    #pragma unroll
        for (int j = 0; j < N; ++j)
    #pragma unroll
          for (int e = 0; e < EPL; ++e) acc[j][e] = 0.f;
        n0 = issue(0, k0, v0);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kRing == 3) n1 = issue(1, k1, v1);
        __builtin_amdgcn_sched_barrier(0);
      }

    }
    if (!split) break;

    // ---- arrivals of this unit's pieces -------------------------------------------
    // Publication: every wave waits until its piece stores (device-coherent
    // atomic stores) are complete, then the workgroup barrier, then thread 0
    // counts the pieces with an agent-scope add; the add therefore reaches
    // memory after every piece store of the workgroup.  Acquisition: the
    // workgroup whose add completes a pair runs an agent-scope acquire fence
    // before the barrier that releases its threads to the merge, whose loads
    // are device-coherent atomic loads.  The add itself is relaxed: an
    // agent-scope release would add an L2 write-back (buffer_wbl2) per
    // workgroup, which publishes plain stores this protocol does not use and
    // cost 15 us a call on the 64-sequence random-length batch.  The last
    // arrival of a pair merges its pieces and leaves the counter at zero for
    // the next call.
    if (pa_s >= 0 || pb_s >= 0) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      // work position of the pair's block 0; its work range starts C earlier
      auto pair_start = [&](int q, int g) { return Hkv * sm_pre[q] + g * cost_of(q) + C; };
      auto pieces = [&](int q, int g) {
        const int A = pair_start(q, g);
        return up.of(A + nb_of(q) - 1) - up.of(A) + 1;
      };
      if (tid == 0) {
        int last_a = 0, last_b = 0;
        if (pa_s >= 0)
          last_a = __hip_atomic_fetch_add(a.counters + pa_s * Hkv + pa_g, 1, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT) == pieces(pa_s, pa_g) - 1;
        if (pb_s >= 0)
          last_b = __hip_atomic_fetch_add(a.counters + pb_s * Hkv + pb_g, 1, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT) == pieces(pb_s, pb_g) - 1;
        if (last_a | last_b) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        sm_last[0] = last_a;
        sm_last[1] = last_b;
      }
      __syncthreads();
      if (sm_last[0]) {
        const int A = pair_start(pa_s, pa_g);
        merge_pair<T, D, N, kThreads>(a, pa_s, pa_g, A - C, A, A + nb_of(pa_s), up, tid);
        if (tid == 0)
          __hip_atomic_store(a.counters + pa_s * Hkv + pa_g, 0, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
      if (sm_last[1]) {
        const int A = pair_start(pb_s, pb_g);
        merge_pair<T, D, N, kThreads>(a, pb_s, pb_g, A - C, A, A + nb_of(pb_s), up, tid);
        if (tid == 0)
          __hip_atomic_store(a.counters + pb_s * Hkv + pb_g, 0, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
    }

    // ---- the next unit: a chunk, while there are any ----------------------------
    if (up.U == up.G) break;
    if (tid == 0)
      sm_unit = up.G + __hip_atomic_fetch_add(ctl, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    u = sm_unit;
    __syncthreads();
    if (u >= up.U) break;
  }
  // ---- kStep: the new token of sequences blockIdx.x, + grid, ... to its slot,
  // by pa_append_kv's rule (position L - 1 of the raw length; none for an
  // empty context, a position past the table, or an entry outside the pool).
  // Nothing in the call reads these rows, so the workgroup writes them when
  // its own units are done, off the path of its first loads.
  if constexpr (kStep) {
    const uint32_t bsh = a.geom.block_shift;
    const int head_bytes_ = D * static_cast<int>(sizeof(T));
    const int chunks = a.num_kv_heads * head_bytes_ / 16;     // 16-byte chunks of one row
    for (int q = blockIdx.x; q < S; q += gridDim.x) {
      const int pos = a.context_lens[q] - 1;
      int64_t slot = -1;
      if (pos >= 0 && (pos >> bsh) < a.max_blocks_per_seq) {
        const int phys =
            a.block_tables[static_cast<int64_t>(q) * a.max_blocks_per_seq + (pos >> bsh)];
        if (phys >= 0 && phys < a.num_blocks)
          slot = (static_cast<int64_t>(phys) << bsh) + (pos & ((1 << bsh) - 1));
      }
      if (tid == 0 && a.slot_mapping != nullptr) a.slot_mapping[q] = slot;
      for (int i = tid; slot >= 0 && i < 2 * chunks; i += kThreads) {
        const bool is_v = i >= chunks;
        const int c = is_v ? i - chunks : i;
        const int hh = c / (head_bytes_ / 16);
        const int cq = c - hh * (head_bytes_ / 16);
        const uint4 val = reinterpret_cast<const uint4*>(is_v ? a.v_new : a.k_new)
            [static_cast<int64_t>(q) * chunks + c];
        const int64_t blk = slot >> bsh;
        const int64_t dst = blk * a.geom.block_stride +
                            static_cast<int64_t>(slot - (blk << bsh)) * a.geom.token_stride +
                            static_cast<int64_t>(hh) * a.geom.head_stride + 16 * cq;
        char* pool = static_cast<char*>(const_cast<void*>(is_v ? a.v_cache : a.k_cache));
        *reinterpret_cast<uint4*>(pool + dst) = val;
      }
    }
  }

  // the last workgroup to finish leaves both counters at zero for the next call
  // (every other workgroup has taken its last unit by then)
  if (split && up.U > up.G && tid == 0) {
    if (__hip_atomic_fetch_add(ctl + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
        static_cast<int>(gridDim.x) - 1) {
      __hip_atomic_store(ctl, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(ctl + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// The persistent grid: what the device holds at once, but no more
// workgroups than there are slices (split) or pairs (whole pairs).
template <typename T, int D, int R, bool kSmall, bool kStep>
hipError_t grid_typed(const DecodeArgs& a, int* grid) {
  const size_t lds = plan_lds_bytes(a.num_seqs);
  const void* fn = reinterpret_cast<const void*>(&decode_kernel<T, D, R, kSmall, kStep>);
  int resident = 0;
  constexpr int kThreads = 64 * decode_waves<T, D, R>();
  hipError_t e = resident_workgroups(fn, kThreads, lds, &resident);
  if (e != hipSuccess) return e;
  const int64_t work = a.min_slice_blocks > 0
                           ? static_cast<int64_t>(a.max_slices)
                           : static_cast<int64_t>(a.num_kv_heads) * a.num_seqs;
  *grid = static_cast<int>(resident < work ? resident : (work > 0 ? work : 1));
  return hipSuccess;
}

template <typename T, int D, int R, bool kSmall, bool kStep>
hipError_t run_typed(const DecodeArgs& a, hipStream_t stream, int* grid_only) {
  int grid = 0;
  const hipError_t e = grid_typed<T, D, R, kSmall, kStep>(a, &grid);
  if (e != hipSuccess) return e;
  if (grid_only != nullptr) {
    *grid_only = grid;
    return hipSuccess;
  }
  constexpr int kThreads = 64 * decode_waves<T, D, R>();
  return launch_kernel(decode_kernel<T, D, R, kSmall, kStep>, dim3(grid), dim3(kThreads),
                       plan_lds_bytes(a.num_seqs), stream, a);
}

template <typename T, int D, bool kSmall, bool kStep>
hipError_t run_heads_step(const DecodeArgs& a, hipStream_t stream, int* grid_only) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return run_typed<T, D, 0, kSmall, kStep>(a, stream, grid_only);
    case 2: return run_typed<T, D, 1, kSmall, kStep>(a, stream, grid_only);
    case 4: return run_typed<T, D, 2, kSmall, kStep>(a, stream, grid_only);
    case 8: return run_typed<T, D, 3, kSmall, kStep>(a, stream, grid_only);
    default: return hipErrorInvalidValue;
  }
}

// pa_decode_step (k_new set) runs the kStep variant
template <typename T, int D, bool kSmall>
hipError_t run_heads(const DecodeArgs& a, hipStream_t stream, int* grid_only) {
  return a.k_new != nullptr ? run_heads_step<T, D, kSmall, true>(a, stream, grid_only)
                            : run_heads_step<T, D, kSmall, false>(a, stream, grid_only);
}

// Blocks of 8 tokens hold half a 16-token unit: a variant of their own.
template <typename T, int D>
hipError_t run_blocks(const DecodeArgs& a, hipStream_t stream, int* grid_only) {
  return a.geom.block_shift < 4 ? run_heads<T, D, true>(a, stream, grid_only)
                                : run_heads<T, D, false>(a, stream, grid_only);
}

// Launch the decode, or with grid_only set only report the grid it would use.
hipError_t run(const DecodeArgs& a, hipStream_t stream, int* grid_only) {
  if (a.dtype == 1) {
    if (a.head_dim == 128) return run_blocks<uint16_t, 128>(a, stream, grid_only);
    if (a.head_dim == 64) return run_blocks<uint16_t, 64>(a, stream, grid_only);
  } else {
    if (a.head_dim == 128) return run_blocks<float, 128>(a, stream, grid_only);
    if (a.head_dim == 64) return run_blocks<float, 64>(a, stream, grid_only);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  return run(a, stream, nullptr);
}

hipError_t decode_grid(const DecodeArgs& a, int* grid) { return run(a, nullptr, grid); }

}  // namespace pa
