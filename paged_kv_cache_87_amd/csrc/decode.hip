// Paged-attention decode for gfx950: one query row per (sequence, query
// head) against the sequence's whole history, read block by block through
// its block table, with an online (running max / running sum) softmax
// (JuliaPagedAttn README, "Online Softmax" and "API Reference":
// paged_attention_cpu!; nanoserve Day 19, "What I added today": attend over
// the whole history through the block table in place).
//
// Work decomposition
//   grid (partition, kv_head, sequence), 256 threads = 4 waves.  A
//   partition is `partition_size` consecutive tokens (whole blocks); the
//   waves of a workgroup take the partition's blocks round-robin.
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
// End of a workgroup: rows and then waves are merged with the same
// max/sum rescaling; a sequence that fits in one partition is normalised and
// written to `out`, otherwise the partition's (m, l, o/l) go to the
// workspace and merge_kernel combines partitions by log-sum-exp weights.

#include <float.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kNegBig = -1.0e30f;  // "no score yet": finite, so m - m stays 0

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

template <typename T, int D, int R>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  using LT = Layout<T, D>;
  constexpr int N = 1 << R;          // query heads per KV head
  constexpr int W = 16 >> R;         // lanes per head after the reduce-scatter
  constexpr int EPL = LT::kEPL;
  constexpr int NW = LT::kNW;
  using F = Frag<NW>;

  __shared__ float sm_acc[kWaves][N][D];
  __shared__ float sm_m[kWaves][N];
  __shared__ float sm_l[kWaves][N];

  const int part = blockIdx.x;
  const int g = blockIdx.y;
  const int s = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63;
  const int row = lane >> 4;
  const int li = lane & 15;

  int L = a.context_lens[s];
  L = L < 0 ? 0 : (L > a.context_cap ? a.context_cap : L);
  const int P = a.partition_size;
  const int npart = L > 0 ? (L + P - 1) / P : 1;
  if (part >= npart) return;
  const int tok0 = part * P;
  const int tok1 = (tok0 + P < L) ? tok0 + P : L;
  const int blk0 = tok0 / kBlockSize;
  const int blk1 = (tok1 + kBlockSize - 1) / kBlockSize;

  // ---- query heads of the group, in this lane's scatter order -------------
  const int own = li >> (4 - R);     // head whose full score this lane ends with
  uint32_t qv[N][NW];
  {
    const char* qb = static_cast<const char*>(a.q) +
                     ((static_cast<int64_t>(s) * a.num_q_heads + g * N) * D + li * EPL) * LT::kElt;
#pragma unroll
    for (int idx = 0; idx < N; ++idx) {
      const int h = own ^ scatter_head_xor<R>(idx);
      const F f = load_frag<NW>(qb + static_cast<int64_t>(h) * D * LT::kElt);
#pragma unroll
      for (int w = 0; w < NW; ++w) qv[idx][w] = f.w[w];
    }
  }
  int slot_head[N];                  // head carried by accumulator slot j
  bcast_all_i<R>(own, slot_head);

  float m = kNegBig, l = 0.f;
  float acc[N][EPL];
#pragma unroll
  for (int j = 0; j < N; ++j)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[j][e] = 0.f;

  const int64_t row_bytes = static_cast<int64_t>(a.num_kv_heads) * D * LT::kElt;
  const int64_t block_bytes = row_bytes * kBlockSize;
  const int64_t lane_off = (static_cast<int64_t>(g) * D + li * EPL) * LT::kElt + row * row_bytes;
  const char* kbase = static_cast<const char*>(a.k_cache) + lane_off;
  const char* vbase = static_cast<const char*>(a.v_cache) + lane_off;
  const int32_t* table = a.block_tables + static_cast<int64_t>(s) * a.max_blocks_per_seq;
  const float sl2 = a.scale_log2;

  // Valid tokens of block j (0 when its table entry is not a pool block).
  auto block_valid = [&](int j, int& phys) {
    phys = uniform(table[j]);
    const bool bad = phys < 0 || phys >= a.num_blocks;
    if (bad) phys = 0;
    const int n = tok1 - j * kBlockSize;
    return bad ? 0 : (n < kBlockSize ? n : kBlockSize);
  };

  auto load_block = [&](int phys, F (&kf)[4], F (&vf)[4]) {
    const int64_t off = static_cast<int64_t>(phys) * block_bytes;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      kf[u] = load_frag<NW>(kbase + off + u * 4 * row_bytes);
      vf[u] = load_frag<NW>(vbase + off + u * 4 * row_bytes);
    }
  };

  auto process = [&](F (&kf)[4], F (&vf)[4], int nvalid) {
    float z[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float part_dot[N];
#pragma unroll
      for (int idx = 0; idx < N; ++idx) part_dot[idx] = frag_dot<T, D>(qv[idx], kf[u], 0.f);
      z[u] = reduce_scatter<R>(part_dot) * sl2;
    }
    if (nvalid < kBlockSize) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (row + 4 * u >= nvalid) {
          z[u] = -INFINITY;
#pragma unroll
          for (int w = 0; w < NW; ++w) vf[u].w[w] = 0u;
        }
      }
    }
    const float mx = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    const float m_new = fmaxf(m, mx);
    const float alpha = fast_exp2(m - m_new);
    float p[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) p[u] = fast_exp2(z[u] - m_new);
    l = l * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
    m = m_new;

    float alpha_j[N];
    bcast_all<R>(alpha, alpha_j);
#pragma unroll
    for (int j = 0; j < N; ++j)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[j][e] *= alpha_j[j];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float pj[N];
      bcast_all<R>(p[u], pj);
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float v = frag_elem<T, D>(vf[u], e);
#pragma unroll
        for (int j = 0; j < N; ++j) acc[j][e] = fmaf(pj[j], v, acc[j][e]);
      }
    }
  };

  // ---- main loop: blocks blk0+wave, +4, ... with one block prefetched -----
  {
    F ka[4], va[4], kb[4], vb[4];
    int j = blk0 + wave;
    int phys_a = 0, phys_b = 0, nva = 0, nvb = 0;
    if (j < blk1) {
      nva = block_valid(j, phys_a);
      load_block(phys_a, ka, va);
    }
    while (j < blk1) {
      if (j + kWaves < blk1) {
        nvb = block_valid(j + kWaves, phys_b);
        load_block(phys_b, kb, vb);
      }
      process(ka, va, nva);
      j += kWaves;
      if (j >= blk1) break;
      if (j + kWaves < blk1) {
        nva = block_valid(j + kWaves, phys_a);
        load_block(phys_a, ka, va);
      }
      process(kb, vb, nvb);
      j += kWaves;
    }
  }

  // ---- merge the four rows of the wave -------------------------------------
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
      const float c0 = fast_exp2(ms[j] - mn);
      const float c1 = fast_exp2(mo - mn);
      ls[j] = ls[j] * c0 + lo * c1;
      ms[j] = mn;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[j][e] = acc[j][e] * c0 + __shfl_xor(acc[j][e], off) * c1;
    }
  }

  // ---- merge the waves through LDS -----------------------------------------
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
  __syncthreads();

  const bool direct = npart == 1;
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
    const int qh = g * N + h;
    if (direct) {
      store_out<T>(a.out, (static_cast<int64_t>(s) * a.num_q_heads + qh) * D + d, val);
    } else {
      const int64_t pi = (static_cast<int64_t>(s) * a.num_q_heads + qh) * a.num_partitions + part;
      a.part_o[pi * D + d] = val;
      if (d == 0) {
        a.part_ml[pi * 2 + 0] = M;
        a.part_ml[pi * 2 + 1] = lsum;
      }
    }
  }
}

// Log-sum-exp merge of the partitions of one (sequence, query head):
// out = sum_j w_j o_j / sum_j w_j with w_j = l_j * 2^(m_j - max m).
template <typename T, int D>
__global__ __launch_bounds__(D) void merge_kernel(DecodeArgs a) {
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int d = threadIdx.x;
  int L = a.context_lens[s];
  L = L < 0 ? 0 : (L > a.context_cap ? a.context_cap : L);
  const int npart = L > 0 ? (L + a.partition_size - 1) / a.partition_size : 1;
  if (npart <= 1) return;  // the decode kernel wrote this row itself
  const int64_t base = (static_cast<int64_t>(s) * a.num_q_heads + h) * a.num_partitions;
  float M = kNegBig;
  for (int j = 0; j < npart; ++j) M = fmaxf(M, a.part_ml[(base + j) * 2]);
  float wsum = 0.f, osum = 0.f;
  for (int j = 0; j < npart; ++j) {
    const float w = a.part_ml[(base + j) * 2 + 1] * fast_exp2(a.part_ml[(base + j) * 2] - M);
    wsum += w;
    osum += w * a.part_o[(base + j) * D + d];
  }
  store_out<T>(a.out, (static_cast<int64_t>(s) * a.num_q_heads + h) * D + d,
               wsum > 0.f ? osum / wsum : 0.f);
}

template <typename T, int D, int R>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid(a.num_partitions, a.num_kv_heads, a.num_seqs);
  hipLaunchKernelGGL((decode_kernel<T, D, R>), grid, dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_partitions == 1) return e;
  hipLaunchKernelGGL((merge_kernel<T, D>), dim3(a.num_q_heads, a.num_seqs), dim3(D), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_heads(const DecodeArgs& a, hipStream_t stream) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_typed<T, D, 0>(a, stream);
    case 2: return launch_typed<T, D, 1>(a, stream);
    case 4: return launch_typed<T, D, 2>(a, stream);
    case 8: return launch_typed<T, D, 3>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.dtype == 1) {
    if (a.head_dim == 128) return launch_heads<uint16_t, 128>(a, stream);
    if (a.head_dim == 64) return launch_heads<uint16_t, 64>(a, stream);
  } else {
    if (a.head_dim == 128) return launch_heads<float, 128>(a, stream);
    if (a.head_dim == 64) return launch_heads<float, 64>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
