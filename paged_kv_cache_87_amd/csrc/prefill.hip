// Batched causal prefill for gfx950 on bf16 matrix cores (head_dim 64 or 128):
// every new token of every sequence attends to its paged history up to and
// including its own position, all in one launch (JuliaPagedAttn README, "Features": batched
// prefill, all prompt positions in a single kernel call; "Online Softmax").
//
// Work decomposition
//   a one-dimensional grid, 8 x ceil(pairs / 8) x (query tiles of the
//   longest prompt) workgroups, mapped to (query tile, KV head, sequence)
//   die by die (see the kernel), 256 threads = 4 waves.  A tile has
//   128 columns = (query head of the GQA group, token) pairs: 128 / n_rep
//   consecutive new tokens of the sequence times the n_rep query heads that
//   share the KV head (GQA, nanoserve Day 19 "What I learned" item 4), so a
//   K/V tile brought into LDS serves every head of the group.  Wave w owns
//   columns 32w .. 32w+31.
//   The keys are walked in tiles of 32 (two 16-token blocks, each found
//   through the block table) up to the tile's last position; K and V are
//   staged in LDS as [key][d] rows, double-buffered: at the start of a tile
//   the next tile's K/V (loaded during the previous tile) are stashed and
//   the loads of the tile after that are issued, so every load has a whole
//   tile of math to arrive.  32-key tiles keep the kernel at 162 VGPRs and
//   39 KB of LDS, so three workgroups (three waves per SIMD) share a CU; with
//   64-key tiles it needed 198 VGPRs and 70 KB, two per CU, and ran ~6 %
//   slower.
//
// Arithmetic (v_mfma_f32_32x32x16_bf16, fp32 accumulation)
//   S^T = K . Q^T   : keys on the M axis, the wave's 32 columns on N; the
//                     softmax reductions over keys are then mostly inside a
//                     lane (16 keys per lane per 32-key tile) plus one swap
//                     between the two lane halves.
//   O^T += V^T . P^T: the accumulator layout of S^T, rounded to bf16, is
//                     directly the B operand of the P.V product when the
//                     contraction index k of lane half h is mapped to key
//                     16c + 4h + (k mod 4) + 8 (k div 4) for 16-key step c.
//                     The V^T fragments (four consecutive keys of one d per
//                     read) come from the [key][d] rows through gfx950's
//                     transposing LDS read: in each 16-lane group, source
//                     lane s addresses key row s/4 and d columns 4 (s mod 4)
//                     .. +3, and lane i receives d column i of the four rows.
//   Online softmax per column (running max / running sum) on the raw scores,
//   scaled inside the exponent; the causal mask is applied only on the key
//   tiles that reach past a column's position.  The reference max only moves
//   when a score passes it by more than 2^8 (then O is rescaled).

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kPWaves = 4;
constexpr int kPThreads = 64 * kPWaves;
constexpr int kCols = 128;            // (head, token) columns per workgroup
constexpr int kKeys = 32;             // keys per K/V tile (2 blocks)
constexpr int kHalves = kKeys / 32;   // 32-key halves per tile = loader passes
// LDS row strides of K and V (bf16 elements), for gfx950's 64 banks of 4 bytes:
// a K fragment read (16 bytes per lane) serves 16 key rows at a time, which a
// stride of D/2 + 4 dwords spreads over all 64 banks; a transposing V read (8
// bytes per lane) serves 4 key rows x 64 bytes at a time, which need rows 16
// banks apart: D/2 + 16 dwords (80 at head_dim 128, 48 at 64)
template <int D> constexpr int kKStride = D + 8;
template <int D> constexpr int kVStride = D + 32;
constexpr float kPNegBig = -1.0e30f;
constexpr float kPRescale = 8.f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// 16-byte aligned, so that the tile rows are read and written with 16-byte
// LDS instructions
template <int D>
struct alignas(16) PrefillSmem {
  uint16_t k[2][kKeys][kKStride<D>];  // K tile, [key][d]
  uint16_t v[2][kKeys][kVStride<D>];  // V tile, [key][d]
  uint32_t bad[2];                    // byte w: wave w's 8-key group of the tile is not in the pool
};

// The q / out rows of sequence s: [q0, q0 + q_len), q_start_loc clamped to
// [0, total_q_tokens] so that no row outside the buffers is touched.
__device__ __forceinline__ void seq_rows(const PrefillArgs& a, int s, int& q0, int& q_len) {
  int lo = a.q_start_loc[s];
  int hi = a.q_start_loc[s + 1];
  lo = min(max(lo, 0), a.total_q_tokens);
  hi = min(max(hi, lo), a.total_q_tokens);
  q0 = lo;
  q_len = hi - lo;
}

// x of lane ^ 32 through the gfx950 lane-half swap (no LDS round trip)
__device__ __forceinline__ float xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f32x2 two = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(two, bf16x2));
}

// ---- which tile: the dies take (sequence, KV head) pairs round-robin -------
// Workgroups are handed to the eight dies (XCDs) round-robin by linear id,
// so linear id i runs on die i mod 8.  Die x works through the pairs x,
// x + 8, x + 16, ... one after the other, each pair's tiles heaviest first:
// every tile of a pair then runs on the die whose L2 already holds the
// pair's K/V, and with eight KV heads each die gets one head of every
// sequence, the same work.  The grid is an upper bound; surplus workgroups
// find no tile (sm_pick[0] < 0) and leave.  Otherwise sm_pick holds the
// sequence, the KV head and the tile's place among the pair's tiles
// (0 = the heaviest).  TQ is the tokens per tile.
__device__ __forceinline__ void pick_tile(const PrefillArgs& a, int TQ, int* sm_scan,
                                          int* sm_pick) {
  const int tid = threadIdx.x;
  const int lin = blockIdx.x;
  const int die = lin & 7;
  const int want = lin >> 3;                    // index in this die's queue of tiles
  const int npairs = a.num_seqs * a.num_kv_heads;
  const int mine = (npairs - die + 7) / 8;      // pairs die, die + 8, ...
  if (tid == 0) sm_pick[0] = -1;
  __syncthreads();
  int base = 0;                                 // tiles of the die's earlier chunks
  for (int c0 = 0; c0 < mine; c0 += kPThreads) {
    int nt = 0;
    if (c0 + tid < mine) {
      const int ss = (die + 8 * (c0 + tid)) / a.num_kv_heads;
      int q0, ql;
      seq_rows(a, ss, q0, ql);
      nt = (min(ql, a.max_q_len) + TQ - 1) / TQ;
    }
    // inclusive scan of the chunk's tile counts (Hillis-Steele in LDS)
    sm_scan[tid] = nt;
    __syncthreads();
    for (int off = 1; off < kPThreads; off <<= 1) {
      const int y = tid >= off ? sm_scan[tid - off] : 0;
      __syncthreads();
      sm_scan[tid] += y;
      __syncthreads();
    }
    const int incl = base + sm_scan[tid];
    if (nt > 0 && want < incl && want >= incl - nt) {
      const int p = die + 8 * (c0 + tid);
      sm_pick[0] = p / a.num_kv_heads;
      sm_pick[1] = p - sm_pick[0] * a.num_kv_heads;
      sm_pick[2] = want - (incl - nt);            // place among the pair's tiles
    }
    base += sm_scan[kPThreads - 1];
    __syncthreads();
    if (sm_pick[0] >= 0 || want < base) break;
  }
}

template <int R, int kD>
__global__ __launch_bounds__(kPThreads) void prefill_kernel(PrefillArgs a) {
  static_assert(kD == 64 || kD == 128, "head_dim 64 or 128");
  constexpr int NREP = 1 << R;
  constexpr int TQ = kCols / NREP;    // tokens per tile
  constexpr int kCPR = kD / 8;        // 16-byte chunks per K/V row
  constexpr int kEPW = kCPR / 8;      // keys per lane and pass in the loader (2 or 1)
  __shared__ PrefillSmem<kD> sm;

  const int tid = threadIdx.x;
  __shared__ int sm_scan[kPThreads];
  __shared__ int sm_pick[3];
  pick_tile(a, TQ, sm_scan, sm_pick);
  if (sm_pick[0] < 0) return;
  const int s = sm_pick[0];
  const int g = sm_pick[1];
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63;
  const int half = lane >> 5;         // lane half: rows 4*half.. of each 8-row group
  const int col = lane & 31;          // this lane's column inside the wave

  // The sequence's q_len new tokens sit at positions L - q_len .. L - 1.  The
  // newest n_q = min(q_len, max_q_len) of them are computed, each at its own
  // position (older rows are not written); a token whose position is
  // negative sees no key and gets a zero row.
  int qs0, q_len;
  seq_rows(a, s, qs0, q_len);
  int L = a.context_lens[s];
  L = L < 0 ? 0 : (L > a.context_cap ? a.context_cap : L);
  const int n_q = min(q_len, a.max_q_len);
  const int row0 = qs0 + q_len - n_q;  // q / out row of computed token 0
  const int n_tiles = (n_q + TQ - 1) / TQ;
  const int tile = n_tiles - 1 - sm_pick[2];      // heaviest tiles (most keys) first
  if (tile < 0) return;
  const int t0 = tile * TQ;
  const int first_pos = L - n_q;      // position of computed token 0 (may be negative)

  // ---- this lane's column: (head, token) ----------------------------------
  const int c = wave * 32 + col;
  const int head = c / TQ;
  const int tok = t0 + c % TQ;
  const bool col_valid = tok < n_q;
  const int qpos = first_pos + tok;   // the column's query position
  const int qh = g * NREP + head;

  // Q^T as B operand: lane holds q[d = 16*kk + 8*half + 0..7] for kk = 0..7
  bf16x8 qf[kD / 16];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           (static_cast<int64_t>(row0 + (col_valid ? tok : 0)) * a.num_q_heads + qh) * kD;
#pragma unroll
    for (int kk = 0; kk < kD / 16; ++kk) {
      uint4 x = *reinterpret_cast<const uint4*>(qrow + 16 * kk + 8 * half);
      if (!col_valid) x = make_uint4(0u, 0u, 0u, 0u);
      qf[kk] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // last key any column of the tile needs
  const int last_tok = min(t0 + TQ, n_q) - 1;
  const int key_end = first_pos + last_tok + 1;       // keys [0, key_end)
  const int n_kt = key_end > 0 ? (key_end + kKeys - 1) / kKeys : 0;
  const int32_t* table = a.block_tables + static_cast<int64_t>(s) * a.max_blocks_per_seq;
  const uint32_t row_bytes = a.geom.token_stride;     // next token row of one KV head
  const uint32_t block_bytes = a.geom.span;           // a block's rows (both layouts)

  // ---- K/V tile loader: kKeys keys x kD d, K and V as [key][d] rows ---------
  // thread -> (keys 8 w + kEPW (lane / kCPR) + 0 .. kEPW - 1 (+32 per further
  // pass), d chunk dc = lane % kCPR): wave w loads keys 8 w .. 8 w + 7 of a
  // pass, so the keys of one wave and pass lie in one 16-token block,
  // so its block id is wave-uniform and the loads go through a buffer
  // descriptor; keys past the context read as zeros (offset past the
  // descriptor's size), so no pool row outside the context reaches the P.V.
  // A table entry that is not a block of the pool loads zeros too, and the
  // wave records it in its byte of the tile's flag word (`bad`) so that those
  // keys get no weight, as the decode skips such blocks.  Only a tile that
  // reaches past the context needs the per-lane past-the-end offsets.
  const int ld_key = 8 * wave + kEPW * (lane / kCPR);   // first of the lane's keys
  const int ld_dc = lane % kCPR;                         // 8-element chunk of d
  // offset of the lane's first key and chunk from the wave's first key (the
  // wave's 8 keys are consecutive rows of one block at any block size >= 8)
  const uint32_t ld_off = (ld_key - 8 * wave) * row_bytes + g * a.geom.head_stride + ld_dc * 16;
  const uint32_t bshift = a.geom.block_shift;
  const char* kpool = static_cast<const char*>(a.k_cache);
  const char* vpool = static_cast<const char*>(a.v_cache);
  auto load_ids = [&](int kt, int (&ids)[kHalves]) {
#pragma unroll
    for (int ps = 0; ps < kHalves; ++ps) {
      const int kpos0 = kt * kKeys + 8 * wave + 32 * ps;   // the wave's first key this pass
      ids[ps] = kpos0 < L ? table[kpos0 >> bshift] : -1;
    }
  };
  uint4 kreg[kHalves][kEPW], vreg[kHalves][kEPW];  // [pass][key of the lane's run]
  int kbad[kHalves];                                // the pass's block is not in the pool
  auto fetch = [&](int kt, const int (&ids)[kHalves]) {
#pragma unroll
    for (int ps = 0; ps < kHalves; ++ps) {
      const int phys = uniform(ids[ps]);
      const bool ok = phys >= 0 && phys < a.num_blocks;
      kbad[ps] = ok ? 0 : 1;
      const int kpos0 = kt * kKeys + 8 * wave + 32 * ps;    // the wave's first key
      const uint32_t sub_bytes =
          static_cast<uint32_t>(kpos0 & ((1 << bshift) - 1)) * row_bytes;
      const int64_t boff = ok ? static_cast<int64_t>(phys) * a.geom.block_stride + sub_bytes : 0;
      const uint32_t size = ok ? block_bytes - sub_bytes : 0u;
      const Rsrc rk = make_rsrc(kpool + boff, size);
      const Rsrc rv = make_rsrc(vpool + boff, size);
#pragma unroll
      for (int e = 0; e < kEPW; ++e) {
        const int kpos = kt * kKeys + ld_key + 32 * ps + e;
        const bool whole = kt * kKeys + kKeys <= L;       // the tile lies inside the context
        const uint32_t off = (whole || kpos < L) ? ld_off + e * row_bytes : size;
        typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 kx = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
        const u32x4 vx = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
        kreg[ps][e] = make_uint4(kx[0], kx[1], kx[2], kx[3]);
        vreg[ps][e] = make_uint4(vx[0], vx[1], vx[2], vx[3]);
      }
    }
  };
  uint16_t* const kst = &sm.k[0][ld_key][ld_dc * 8];
  uint16_t* const vst = &sm.v[0][ld_key][ld_dc * 8];
  auto stash = [&](int buf) {
#pragma unroll
    for (int ps = 0; ps < kHalves; ++ps) {
#pragma unroll
      for (int e = 0; e < kEPW; ++e) {
        const int r = 32 * ps + e;
        *reinterpret_cast<uint4*>(kst + buf * (kKeys * kKStride<kD>) + r * kKStride<kD>) = kreg[ps][e];
        *reinterpret_cast<uint4*>(vst + buf * (kKeys * kVStride<kD>) + r * kVStride<kD>) = vreg[ps][e];
      }
      // wave w loads the tile's keys 8 w .. 8 w + 7: byte w of the tile's flag word
      reinterpret_cast<uint8_t*>(&sm.bad[buf])[wave] = static_cast<uint8_t>(kbad[ps]);
    }
  };
  // transposing-read source address of this lane: key row 4 * half + (lane % 16) / 4,
  // d column 16 * (lane / 16 mod 2) + 4 * (lane mod 4) (plus the step's offsets)
  const int tr_row = 4 * half + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  f32x16 o[kD / 32];                  // O^T: kD / 32 d-tiles of 32 x (32 columns)
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m = kPNegBig, lsum = 0.f;
  const float sl2 = a.scale_log2;
  // the tile's smallest query position: key tiles up to it need no mask
  const int min_qpos = first_pos + t0;

  int ids[kHalves];
  if (n_kt > 0) {
    load_ids(0, ids);
    fetch(0, ids);
    stash(0);
    if (n_kt > 1) {
      load_ids(1, ids);
      fetch(1, ids);
      if (n_kt > 2) load_ids(2, ids);
    }
  }
  __syncthreads();
  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt & 1;
    // Tile kt + 1 was fetched at the start of the previous tile: stash it
    // first (buffer buf^1 was last read before the previous barrier), then
    // issue tile kt + 2's loads into the same registers.  With the stash
    // ahead of the new loads, its wait covers only loads a whole tile old.
    if (kt + 1 < n_kt) {
      stash(buf ^ 1);
      if (kt + 2 < n_kt) {
        fetch(kt + 2, ids);
      }
    }

    // ---- S^T = K . Q^T for every 32-key half of the tile first (with 64-key
    // tiles the second half's matrix work then runs under the first half's
    // softmax) -----------------------------------------------------------------
    f32x16 st[kHalves];
#pragma unroll
    for (int t = 0; t < kHalves; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st[t][r] = 0.f;
      // K fragments two products ahead, the order pinned: each product waits
      // only for a read issued two products earlier (~2 % over the
      // compiler's own order, which waited on each pair of reads)
      constexpr int kAhead = 2;
      uint4 kq[kD / 16];
#pragma unroll
      for (int kk = 0; kk < kAhead; ++kk)
        kq[kk] = *reinterpret_cast<const uint4*>(&sm.k[buf][32 * t + col][16 * kk + 8 * half]);
#pragma unroll
      for (int kk = 0; kk < kD / 16; ++kk) {
        st[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kq[kk]), qf[kk],
                                                         st[t], 0, 0, 0);
        if (kk + kAhead < kD / 16)
          kq[kk + kAhead] = *reinterpret_cast<const uint4*>(
              &sm.k[buf][32 * t + col][16 * (kk + kAhead) + 8 * half]);
      }
      // schedule: kAhead LDS reads (mask 0x100), then one product (0x008) and
      // one read at a time
      __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
      for (int kk = 0; kk < kD / 16; ++kk) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (kk + kAhead < kD / 16) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    // ---- per half: causal mask, online softmax, O^T += V^T . P^T ------------
#pragma unroll
    for (int t = 0; t < kHalves; ++t) {
      // causal mask only where the half reaches past a position; lanes of
      // invalid columns compute values that are never stored
      const int key0 = kt * kKeys + 32 * t;
      if (key0 + 31 > min_qpos) {
        const int lim = qpos - key0 - 4 * half;   // r-part of the key offset must not exceed it
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (8 * (r >> 2) + (r & 3) > lim) st[t][r] = -INFINITY;
      }
      // keys of a block whose table entry is not in the pool get no weight
      const uint32_t bad = static_cast<uint32_t>(uniform(static_cast<int>(sm.bad[buf])));
      if (bad) {
        // accumulator entry r holds a key of the group r / 4
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if ((bad >> (8 * (r >> 2))) & 0xffu) st[t][r] = -INFINITY;
      }
      float tmax = st[t][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, st[t][r]);
      tmax = fmaxf(tmax, xor32(tmax)) * sl2;
      if (__builtin_amdgcn_ballot_w64(tmax > m + kPRescale) != 0) {
        const float m_new = tmax > m + kPRescale ? tmax : m;
        const float alpha = fast_exp2(m - m_new);
        m = m_new;
        lsum *= alpha;
#pragma unroll
        for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
      }
      // P^T in bf16, packed straight from the accumulator layout; the running
      // sum adds the same rounded values the P.V product weights V by (one
      // v_dot2_f32_bf16 against (1, 1) per pair), so the normalised output is
      // a convex combination of the V rows
      uint32_t pk[8];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = fast_exp2(fmaf(st[t][r], sl2, -m));
        const float p1 = fast_exp2(fmaf(st[t][r + 1], sl2, -m));
        pk[r >> 1] = pack_bf16(p0, p1);
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[r >> 1]),
                                               __builtin_bit_cast(bf16x2, 0x3f803f80u), lsum, false);
      }
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
        const int cstep = 2 * t + ch;   // 16-key step of the tile
        const bf16x8 pf = __builtin_bit_cast(
            bf16x8, make_uint4(pk[4 * ch], pk[4 * ch + 1], pk[4 * ch + 2], pk[4 * ch + 3]));
        // keys 16c + 4 half + 0..3 and + 8..11 of d column 32 dt + lane % 32
        const int row = 16 * cstep + tr_row;
#pragma unroll
        for (int dt = 0; dt < kD / 32; ++dt) {
          const int dcol = 32 * dt + tr_col;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4*)&sm.v[buf][row][dcol]);
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4*)&sm.v[buf][row + 8][dcol]);
          const uint2 l2 = __builtin_bit_cast(uint2, lo);
          const uint2 h2 = __builtin_bit_cast(uint2, hi);
          const bf16x8 vx = __builtin_bit_cast(bf16x8, make_uint4(l2.x, l2.y, h2.x, h2.y));
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vx, pf, o[dt], 0, 0, 0);
        }
      }
    }
    // block ids two tiles ahead: read from the table after the products, so the
    // scalar load's wait does not hold up the K fragment reads of this tile
    if (kt + 3 < n_kt) load_ids(kt + 3, ids);
    __syncthreads();
  }

  // ---- normalise and store: lane holds column `col`, rows d ----------------
  lsum += xor32(lsum);
  if (!col_valid) return;
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  uint16_t* orow = static_cast<uint16_t*>(a.out) +
                   (static_cast<int64_t>(row0 + tok) * a.num_q_heads + qh) * kD;
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = 32 * dt + 8 * r4 + 4 * half;
      const uint2 w = make_uint2(pack_bf16(o[dt][4 * r4] * inv, o[dt][4 * r4 + 1] * inv),
                                 pack_bf16(o[dt][4 * r4 + 2] * inv, o[dt][4 * r4 + 3] * inv));
      *reinterpret_cast<uint2*>(orow + d) = w;
    }
}

// ---------------------------------------------------------------------------
// fp32 pools: the same tiles and schedule on the fp32 matrix cores
// (v_mfma_f32_32x32x2_f32), with nothing rounded below fp32.
//   S^T = K . Q^T : contraction step c takes d = c in the lower lane half and
//                   d = c + D/2 in the upper one, so a lane reads its key's
//                   K values four steps at a time from one LDS row and holds
//                   one contiguous half of its column's q row.
//   O^T += V^T . P^T: step r pairs the keys a = 8 (r / 4) + (r mod 4) (lower
//                   half) and a + 4 (upper half), exactly the two keys whose
//                   scores the lane holds in accumulator entry r, so P needs
//                   no move; the lane reads V[its key][d] from LDS.
// ---------------------------------------------------------------------------
template <int D>
struct alignas(16) PrefillSmemF32 {
  // K rows D + 4 floats apart: a 16-byte fragment read serves 16 key rows at
  // a time, 4 banks apart over all 64.  V rows D + 8 apart: a V read (one
  // float a lane) serves the two keys 4 rows apart of the lane halves, 32
  // consecutive floats each, which then fall in opposite halves of the banks.
  float k[2][kKeys][D + 4];           // K tile, [key][d]
  float v[2][kKeys][D + 8];           // V tile, [key][d]
  int bad[2][4 * kHalves];
};

template <int R, int kD>
__global__ __launch_bounds__(kPThreads) void prefill_f32_kernel(PrefillArgs a) {
  static_assert(kD == 64 || kD == 128, "head_dim 64 or 128");
  constexpr int NREP = 1 << R;
  constexpr int TQ = kCols / NREP;    // tokens per tile
  constexpr int kCPR = kD / 4;        // 16-byte chunks per K/V row
  constexpr int kEPW = kCPR / 8;      // keys per lane and pass in the loader (4 or 2)
  constexpr int kH = kD / 2;          // d values per lane half
  __shared__ PrefillSmemF32<kD> sm;

  const int tid = threadIdx.x;
  __shared__ int sm_scan[kPThreads];
  __shared__ int sm_pick[3];
  pick_tile(a, TQ, sm_scan, sm_pick);
  if (sm_pick[0] < 0) return;
  const int s = sm_pick[0];
  const int g = sm_pick[1];
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int col = lane & 31;

  int qs0, q_len;
  seq_rows(a, s, qs0, q_len);
  int L = a.context_lens[s];
  L = L < 0 ? 0 : (L > a.context_cap ? a.context_cap : L);
  const int n_q = min(q_len, a.max_q_len);
  const int row0 = qs0 + q_len - n_q;
  const int n_tiles = (n_q + TQ - 1) / TQ;
  const int tile = n_tiles - 1 - sm_pick[2];
  if (tile < 0) return;
  const int t0 = tile * TQ;
  const int first_pos = L - n_q;

  const int c = wave * 32 + col;
  const int head = c / TQ;
  const int tok = t0 + c % TQ;
  const bool col_valid = tok < n_q;
  const int qpos = first_pos + tok;
  const int qh = g * NREP + head;

  // Q^T as B operand: q[d = half * D/2 + c] for c = 0 .. D/2 - 1
  float qf[kH];
  {
    const float* qrow = static_cast<const float*>(a.q) +
                        (static_cast<int64_t>(row0 + (col_valid ? tok : 0)) * a.num_q_heads + qh) * kD +
                        half * kH;
#pragma unroll
    for (int j = 0; j < kH / 4; ++j) {
      float4 x = reinterpret_cast<const float4*>(qrow)[j];
      if (!col_valid) x = make_float4(0.f, 0.f, 0.f, 0.f);
      qf[4 * j] = x.x; qf[4 * j + 1] = x.y; qf[4 * j + 2] = x.z; qf[4 * j + 3] = x.w;
    }
  }

  const int last_tok = min(t0 + TQ, n_q) - 1;
  const int key_end = first_pos + last_tok + 1;
  const int n_kt = key_end > 0 ? (key_end + kKeys - 1) / kKeys : 0;
  const int32_t* table = a.block_tables + static_cast<int64_t>(s) * a.max_blocks_per_seq;
  const uint32_t row_bytes = a.geom.token_stride;
  const uint32_t block_bytes = a.geom.span;

  // loader: as the bf16 kernel, wave w loads keys 8 w .. 8 w + 7 of a tile
  const int ld_key = 8 * wave + kEPW * (lane / kCPR);
  const int ld_dc = lane % kCPR;
  // offset of the lane's first key and chunk from the wave's first key (the
  // wave's 8 keys are consecutive rows of one block at any block size >= 8)
  const uint32_t ld_off = (ld_key - 8 * wave) * row_bytes + g * a.geom.head_stride + ld_dc * 16;
  const uint32_t bshift = a.geom.block_shift;
  const char* kpool = static_cast<const char*>(a.k_cache);
  const char* vpool = static_cast<const char*>(a.v_cache);
  auto load_ids = [&](int kt, int (&ids)[kHalves]) {
#pragma unroll
    for (int ps = 0; ps < kHalves; ++ps) {
      const int kpos0 = kt * kKeys + 8 * wave + 32 * ps;
      ids[ps] = kpos0 < L ? table[kpos0 >> bshift] : -1;
    }
  };
  uint4 kreg[kHalves][kEPW], vreg[kHalves][kEPW];
  int kbad[kHalves];
  auto fetch = [&](int kt, const int (&ids)[kHalves]) {
#pragma unroll
    for (int ps = 0; ps < kHalves; ++ps) {
      const int phys = uniform(ids[ps]);
      const bool ok = phys >= 0 && phys < a.num_blocks;
      kbad[ps] = ok ? 0 : 1;
      const int kpos0 = kt * kKeys + 8 * wave + 32 * ps;    // the wave's first key
      const uint32_t sub_bytes =
          static_cast<uint32_t>(kpos0 & ((1 << bshift) - 1)) * row_bytes;
      const int64_t boff = ok ? static_cast<int64_t>(phys) * a.geom.block_stride + sub_bytes : 0;
      const uint32_t size = ok ? block_bytes - sub_bytes : 0u;
      const Rsrc rk = make_rsrc(kpool + boff, size);
      const Rsrc rv = make_rsrc(vpool + boff, size);
#pragma unroll
      for (int e = 0; e < kEPW; ++e) {
        const int kpos = kt * kKeys + ld_key + 32 * ps + e;
        const uint32_t off = kpos < L ? ld_off + e * row_bytes : size;
        typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 kx = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
        const u32x4 vx = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
        kreg[ps][e] = make_uint4(kx[0], kx[1], kx[2], kx[3]);
        vreg[ps][e] = make_uint4(vx[0], vx[1], vx[2], vx[3]);
      }
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int ps = 0; ps < kHalves; ++ps) {
#pragma unroll
      for (int e = 0; e < kEPW; ++e) {
        const int key = ld_key + 32 * ps + e;
        *reinterpret_cast<uint4*>(&sm.k[buf][key][ld_dc * 4]) = kreg[ps][e];
        *reinterpret_cast<uint4*>(&sm.v[buf][key][ld_dc * 4]) = vreg[ps][e];
      }
      if (lane == 0) sm.bad[buf][wave + 4 * ps] = kbad[ps];
    }
  };

  f32x16 o[kD / 32];
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m = kPNegBig, lsum = 0.f;
  const float sl2 = a.scale_log2;
  const int min_qpos = first_pos + t0;

  int ids[kHalves];
  if (n_kt > 0) {
    load_ids(0, ids);
    fetch(0, ids);
    stash(0);
    if (n_kt > 1) {
      load_ids(1, ids);
      fetch(1, ids);
      if (n_kt > 2) load_ids(2, ids);
    }
  }
  __syncthreads();
  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < n_kt) {
      stash(buf ^ 1);
      if (kt + 2 < n_kt) fetch(kt + 2, ids);
    }
#pragma unroll
    for (int t = 0; t < kHalves; ++t) {
      // ---- S^T = K . Q^T over D / 2 steps
      f32x16 st;
#pragma unroll
      for (int r = 0; r < 16; ++r) st[r] = 0.f;
#pragma unroll
      for (int j = 0; j < kH / 4; ++j) {
        const float4 kx = *reinterpret_cast<const float4*>(&sm.k[buf][32 * t + col][half * kH + 4 * j]);
        st = __builtin_amdgcn_mfma_f32_32x32x2f32(kx.x, qf[4 * j], st, 0, 0, 0);
        st = __builtin_amdgcn_mfma_f32_32x32x2f32(kx.y, qf[4 * j + 1], st, 0, 0, 0);
        st = __builtin_amdgcn_mfma_f32_32x32x2f32(kx.z, qf[4 * j + 2], st, 0, 0, 0);
        st = __builtin_amdgcn_mfma_f32_32x32x2f32(kx.w, qf[4 * j + 3], st, 0, 0, 0);
      }
      // ---- causal mask, keys of blocks outside the pool, online softmax
      const int key0 = kt * kKeys + 32 * t;
      if (key0 + 31 > min_qpos) {
        const int lim = qpos - key0 - 4 * half;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (8 * (r >> 2) + (r & 3) > lim) st[r] = -INFINITY;
      }
      const int4 bad = *reinterpret_cast<const int4*>(&sm.bad[buf][4 * t]);
      if (bad.x | bad.y | bad.z | bad.w) {
        // accumulator entry r holds a key of the group r / 4
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int b = (r >> 2) == 0 ? bad.x : (r >> 2) == 1 ? bad.y : (r >> 2) == 2 ? bad.z : bad.w;
          if (b) st[r] = -INFINITY;
        }
      }
      float tmax = st[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, st[r]);
      tmax = fmaxf(tmax, xor32(tmax)) * sl2;
      if (__builtin_amdgcn_ballot_w64(tmax > m + kPRescale) != 0) {
        const float m_new = tmax > m + kPRescale ? tmax : m;
        const float alpha = fast_exp2(m - m_new);
        m = m_new;
        lsum *= alpha;
#pragma unroll
        for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
      }
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = fast_exp2(fmaf(st[r], sl2, -m));
        lsum += p[r];
      }
      // ---- O^T += V^T . P^T, step r on keys a + 4 half, a = 8 (r / 4) + r mod 4
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * t + 8 * (r >> 2) + (r & 3) + 4 * half;
#pragma unroll
        for (int dt = 0; dt < kD / 32; ++dt)
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(sm.v[buf][key][32 * dt + col], p[r], o[dt],
                                                       0, 0, 0);
      }
    }
    if (kt + 3 < n_kt) load_ids(kt + 3, ids);
    __syncthreads();
  }

  lsum += xor32(lsum);
  if (!col_valid) return;
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  float* orow = static_cast<float*>(a.out) + (static_cast<int64_t>(row0 + tok) * a.num_q_heads + qh) * kD;
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = 32 * dt + 8 * r4 + 4 * half;
      *reinterpret_cast<float4*>(orow + d) =
          make_float4(o[dt][4 * r4] * inv, o[dt][4 * r4 + 1] * inv, o[dt][4 * r4 + 2] * inv,
                      o[dt][4 * r4 + 3] * inv);
    }
}

}  // namespace

template <int D>
hipError_t launch_heads(const PrefillArgs& a, dim3 grid, hipStream_t stream) {
  if (a.dtype == 0) {
    switch (a.num_q_heads / a.num_kv_heads) {
      case 1: return launch_kernel(prefill_f32_kernel<0, D>, grid, dim3(kPThreads), 0, stream, a);
      case 2: return launch_kernel(prefill_f32_kernel<1, D>, grid, dim3(kPThreads), 0, stream, a);
      case 4: return launch_kernel(prefill_f32_kernel<2, D>, grid, dim3(kPThreads), 0, stream, a);
      case 8: return launch_kernel(prefill_f32_kernel<3, D>, grid, dim3(kPThreads), 0, stream, a);
      default: return hipErrorInvalidValue;
    }
  }
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_kernel(prefill_kernel<0, D>, grid, dim3(kPThreads), 0, stream, a);
    case 2: return launch_kernel(prefill_kernel<1, D>, grid, dim3(kPThreads), 0, stream, a);
    case 4: return launch_kernel(prefill_kernel<2, D>, grid, dim3(kPThreads), 0, stream, a);
    case 8: return launch_kernel(prefill_kernel<3, D>, grid, dim3(kPThreads), 0, stream, a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  const int n_rep = a.num_q_heads / a.num_kv_heads;
  const int tq = kCols / n_rep;
  const int64_t tiles = (a.max_q_len + tq - 1) / tq;
  // Die x (workgroups x, x + 8, ...) serves the pairs x, x + 8, ...: at most
  // ceil(pairs / 8) pairs of at most `tiles` tiles each, so every die needs
  // that many workgroups of its own, whatever the pair count mod 8.
  const int64_t pairs = static_cast<int64_t>(a.num_seqs) * a.num_kv_heads;
  const int64_t per_die = (pairs + 7) / 8 * tiles;
  if (per_die <= 0) return hipSuccess;
  if (8 * per_die > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(8 * per_die));
  if (a.head_dim == 128) return launch_heads<128>(a, grid, stream);
  if (a.head_dim == 64) return launch_heads<64>(a, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
