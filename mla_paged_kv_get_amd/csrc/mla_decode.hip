// Paged MLA decode kernels for gfx950 (CDNA4).
//
// What is computed ("What is FlashMLA", topnet.top, installation-and-use
// section, step 3; latent rows as in "Novita AI ... FlashMLA 평가", section
// "MLA란 무엇인가요?"): for every query row of an item, softmax-weighted sums of
// V over the item's keys, with K = the 576-value latent row and V = its first
// 512 values, plus the natural-log LSE of the scaled scores.
//
// How it maps onto the chip:
//  * A persistent grid: workgroup = (worker, row tile).  A worker walks the
//    runs of 64-key tiles the scheduler gave it (see mla_plan.hip).
//  * Every 64-row tile (73,728 B) is copied HBM -> LDS with
//    global_load_lds_dwordx4: one instruction moves 8 rows x 128 B, so each
//    wave instruction reads whole 128-byte lines.  Rows are placed in LDS in
//    8-row x 128-B blocks with an XOR swizzle of the 16-byte chunks, which
//    spreads both the row-fragment reads of QK^T and the transposed reads of
//    PV over the LDS banks.  Two tiles are in flight (double buffer in two
//    distinct LDS arrays, so the compiler does not serialise the copy into one
//    with the reads of the other).
//  * S^T = K Q^T with v_mfma_f32_16x16x32_bf16: A = 16 key rows read from LDS,
//    B = 16 query rows held in registers for the whole run (Q is loaded once
//    per run).  The accumulator gives every lane 4 keys of one query row.
//  * Online softmax in base 2 (scores pre-multiplied by scale*log2(e)); the
//    row max is reduced over the 4 lanes holding a row with two xor-shuffles;
//    row sums stay per lane until the end.
//  * O^T += V^T P^T with the same MFMA: P^T comes straight from the S^T
//    accumulators (the key order inside the contraction is permuted to match),
//    V^T fragments come from LDS through ds_read_b64_tr_b16 (a transposing
//    read: 16 lanes read 4 rows x 16 values and each lane receives one column).
//  * Keys past a sequence's length inside its last page, and sparse padding
//    entries, are loaded from a valid row of the same sequence and masked to
//    -inf, so no value outside the key set (e.g. NaN garbage) is ever read.
//  * Runs covering a whole item write bf16 O and fp32 LSE directly; other
//    runs write fp32 partials that the combine kernel merges (log-sum-exp).
#include "mla_common.h"

#include <math.h>

namespace mla {
namespace {

constexpr float kLn2 = 0.69314718055994530942f;

// XOR pattern of tile row t (bijection on t & 7).
__device__ __forceinline__ int swz(int t) { return ((t & 3) << 1) | ((t >> 2) & 1); }

// LDS byte offset of 16-byte chunk c (0..71) of tile row t (0..63): 8-row x
// 128-byte blocks of 1 KB, block (t / 8, c / 8) at index (t / 8) * 9 + c / 8.
__device__ __forceinline__ int lds_off(int t, int c) {
  return (((t >> 3) * 9 + (c >> 3)) << 10) + ((t & 7) << 7) + (((c & 7) ^ swz(t)) << 4);
}

template <int NR, int NT>
struct Cfg {
  static constexpr int kWaves = NR * NT;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kTpw = 64 / NT;                 // keys per wave per tile
  static constexpr int kSub = kTpw / 16;               // 16-key subtiles per wave
  static constexpr int kRows = 16 * NR;                // query rows per workgroup
  static constexpr int kLoads = 72 / kWaves;           // 1 KB copy instructions per wave per tile
  static constexpr int kLaneRows = (kLoads + 8) / 9;   // tile rows each lane copies
  static_assert(72 % kWaves == 0 && kLoads % 9 == 0, "tile copy must split evenly");
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane i
// receives element i % 4 of the 8-byte words addressed by lanes 4 e + i / 4,
// e = 0..3, i.e. one column of the 4 x 16 block the group points at.
__device__ __forceinline__ bf16x4 read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(p));
}

// Per-run state of one wave.
template <int KSUB>
struct WaveState {
  bf16x8 qf[18];        // B operand of S^T: Q[row][32 ks + 8 g .. + 7]
  floatx4 oacc[32];     // O^T[16 dt + 4 g + i][row]
  float m_run;          // running max (base-2 scaled units)
  float l_lane;         // running sum over this lane's keys
};

template <int NR, int NT>
__global__ __launch_bounds__(64 * NR * NT, 1) void decode_kernel(DecodeArgs a) {
  using C = Cfg<NR, NT>;
  __shared__ __attribute__((aligned(1024))) char s0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char s1[kTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char kvalid[2][64];   // sparse key validity per stage
  __shared__ float red_m[NT][C::kRows];
  __shared__ float red_l[NT][C::kRows];

  // Worker and row tile of this workgroup.  Row tiles of one worker are placed
  // 8 workgroups apart so that they land on the same XCD (workgroups are
  // dealt to the 8 XCDs round-robin) and share its L2 for the common tiles.
  int w, mt;
  if (a.m_tiles == 1) {
    w = blockIdx.x;
    mt = 0;
  } else {
    const int grp = blockIdx.x / (8 * a.m_tiles), rem = blockIdx.x % (8 * a.m_tiles);
    mt = rem >> 3;
    w = grp * 8 + (rem & 7);
  }
  if (w >= a.num_workers) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;      // lane group (k slice of MFMA operands)
  const int li = lane & 15;     // row (query row / key row) inside a 16-block
  const int rg = wave % NR;     // row group of this wave
  const int tg = wave / NR;     // key group of this wave
  const int row = mt * C::kRows + rg * 16 + li;   // query row inside the item (S^T column)
  const bool row_ok = row < a.M;

  const int32_t* prow = a.plan + kPlanWords * (1 + w);
  const int it_first = prow[0], blk_first = prow[1], it_last = prow[2], blk_end = prow[3],
            split_first = prow[4];
  if (it_first < 0) return;

  // LDS read offsets of this lane (see lds_off).
  //  K row fragments: key row t = tg*kTpw + li (+16 u), chunk 4 ks + g.
  const int tk = tg * C::kTpw + li;
  const int k_base = ((tk >> 3) * 9 << 10) + ((tk & 7) << 7);
  const int k_x0 = ((g ^ swz(tk)) << 4);            // even ks: chunk & 7 == g
  const int k_x1 = (((4 + g) ^ swz(tk)) << 4);      // odd ks:  chunk & 7 == 4 + g
  //  V^T transposed reads: source row t = tg*kTpw + 4 g + li / 4 (+16 u),
  //  columns 16 dt + 4 (li & 3) .. + 3, i.e. chunk 2 dt + (li & 3) / 2, half li & 1.
  const int tv = tg * C::kTpw + 4 * g + (li >> 2);
  const int v_base = ((tv >> 3) * 9 << 10) + ((tv & 7) << 7) + ((li & 1) << 3);
  int v_x[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) v_x[d] = (((2 * d + ((li & 3) >> 1)) ^ swz(tv)) << 4);

  // Tile rows this lane copies: t = 8 * (wave * kLoads / 9 + r) + lane / 8.
  int cp_row[C::kLaneRows];
  int cp_swz[C::kLaneRows];
#pragma unroll
  for (int r = 0; r < C::kLaneRows; ++r) {
    cp_row[r] = 8 * (wave * C::kLoads / 9 + r) + (lane >> 3);
    cp_swz[r] = swz(cp_row[r]);
  }

  const char* kv_bytes = reinterpret_cast<const char*>(a.kv);

  for (int item = it_first; item <= it_last; ++item) {
    const bool sparse = a.topk > 0;
    const int b = sparse ? item / a.s_q : item;
    const int L = a.seqlens[b];
    const int len = sparse ? a.topk : L;
    const int nblk = len > 0 ? (len + kPage - 1) / kPage : 0;
    const int lo = item == it_first ? blk_first : 0;
    const int hi = item == it_last ? blk_end : nblk;
    if (lo >= hi) continue;
    const int split = item == it_first ? split_first : 0;
    const int slot0 = a.num_splits[item];
    const int nsplit = a.num_splits[item + 1] - slot0;
    const int32_t* bt_row = a.block_table + (int64_t)b * a.max_blocks;
    const int32_t* idx_row = sparse ? a.indices + (int64_t)item * a.topk : nullptr;
    const bool load = !sparse || L > 0;   // a sparse item of an empty sequence has no keys

    // Key limit of this lane's query row (dense); sparse validity comes from LDS.
    int lim = 0;
    if (row_ok) {
      lim = L;
      if (!sparse && a.causal) lim = L - a.s_q + row / a.h_q + 1;
    }

    // Query fragments of this wave's 16 rows.
    WaveState<C::kSub> st;
    {
      const uint16_t* qrow = a.q + ((int64_t)item * a.M + (row_ok ? row : 0)) * kDqk + 8 * g;
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        bf16x8 v = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks);
        if (!row_ok) v = bf16x8{};
        st.qf[ks] = v;
      }
    }
#pragma unroll
    for (int d = 0; d < 32; ++d) st.oacc[d] = floatx4{0.f, 0.f, 0.f, 0.f};
    st.m_run = -INFINITY;
    st.l_lane = 0.f;

    // Byte offsets of the rows this lane copies for tile `blk`.
    auto tile_rows = [&](int blk, int64_t (&off)[C::kLaneRows], unsigned char* vstage) {
      if (!sparse) {
        const int64_t page = bt_row[blk];
        const int nvalid = min(kPage, L - blk * kPage);
#pragma unroll
        for (int r = 0; r < C::kLaneRows; ++r) {
          const int t = min(cp_row[r], nvalid - 1);
          off[r] = (page * kPage + t) * (int64_t)kRowBytes;
        }
      } else {
#pragma unroll
        for (int r = 0; r < C::kLaneRows; ++r) {
          const int sl = blk * kPage + cp_row[r];
          const int idx = sl < a.topk ? idx_row[sl] : -1;
          const bool ok = sparse_key_valid(idx, L);
          off[r] = cache_row(bt_row, ok ? idx : 0) * (int64_t)kRowBytes;
          if ((lane & 7) == 0) vstage[cp_row[r]] = ok ? 1 : 0;
        }
      }
    };
    auto issue = [&](char* stage, const int64_t (&off)[C::kLaneRows]) {
#pragma unroll
      for (int j = 0; j < C::kLoads; ++j) {
        const int ii = wave * C::kLoads + j;
        const int r = j / 9, cl = j % 9;
        const char* src = kv_bytes + off[r] + cl * 128 + (((lane & 7) ^ cp_swz[r]) << 4);
        __builtin_amdgcn_global_load_lds(MLA_GBL(src), MLA_LDS(stage + ii * 1024), 16, 0, 0);
      }
    };

    // Consume one tile held in `stage` (keys blk*64 .. blk*64 + 63 of the item).
    auto compute = [&](const char* stage, const unsigned char* vstage, int blk) {
      floatx4 sacc[C::kSub];
#pragma unroll
      for (int u = 0; u < C::kSub; ++u) sacc[u] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
#pragma unroll
        for (int u = 0; u < C::kSub; ++u) {
          const int off = k_base + u * (2 * 9 * 1024) + ((ks >> 1) << 10) + ((ks & 1) ? k_x1 : k_x0);
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(stage + off);
          sacc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, st.qf[ks], sacc[u], 0, 0, 0);
        }
      }
      // Scale, mask, running max.
      float x[C::kSub][4];
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < C::kSub; ++u) {
        const int t0 = tg * C::kTpw + 16 * u + 4 * g;       // tile row of element i = 0
        unsigned vb = 0;
        if (sparse) vb = *reinterpret_cast<const unsigned*>(vstage + t0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bool ok;
          if (sparse) ok = row_ok && ((vb >> (8 * i)) & 0xff);
          else ok = blk * kPage + t0 + i < lim;
          x[u][i] = ok ? sacc[u][i] * a.scale_log2 : -INFINITY;
          mx = fmaxf(mx, x[u][i]);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(st.m_run, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(st.m_run - m_use);
      float psum = 0.f;
      float p[C::kSub][4];
#pragma unroll
      for (int u = 0; u < C::kSub; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[u][i] = fast_exp2(x[u][i] - m_use);
          psum += p[u][i];
        }
      st.l_lane = st.l_lane * alpha + psum;
      st.m_run = m_new;
#pragma unroll
      for (int d = 0; d < 32; ++d) st.oacc[d] *= alpha;

      // O^T += V^T P^T.
      if constexpr (C::kSub == 1) {
        bf16x8 pb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pb[i] = (__bf16)p[0][i];
          pb[4 + i] = (__bf16)0.f;
        }
        const char* vrow = stage + v_base;
        const bf16x4 zero4 = {};
#pragma unroll
        for (int dt = 0; dt < 32; ++dt) {
          const int off = ((dt >> 2) << 10) + v_x[dt & 3];
          const bf16x4 v0 = read_tr(vrow + off);
          const bf16x8 va = __builtin_shufflevector(v0, zero4, 0, 1, 2, 3, 4, 5, 6, 7);
          st.oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, st.oacc[dt], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int pr = 0; pr < C::kSub / 2; ++pr) {
          bf16x8 pb;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pb[i] = (__bf16)p[2 * pr][i];
            pb[4 + i] = (__bf16)p[2 * pr + 1][i];
          }
          const char* vrow0 = stage + v_base + (2 * pr) * (2 * 9 * 1024);
          const char* vrow1 = vrow0 + 2 * 9 * 1024;
#pragma unroll
          for (int dt = 0; dt < 32; ++dt) {
            const int off = ((dt >> 2) << 10) + v_x[dt & 3];
            const bf16x4 v0 = read_tr(vrow0 + off);
            const bf16x4 v1 = read_tr(vrow1 + off);
            const bf16x8 va = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
            st.oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, st.oacc[dt], 0, 0, 0);
          }
        }
      }
    };

    // Double-buffered walk over tiles lo .. hi - 1.
    if (load) {
      int64_t off[C::kLaneRows];
      tile_rows(lo, off, kvalid[0]);
      issue(s0, off);
      for (int blk = lo; blk < hi; blk += 2) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (blk + 1 < hi) {
          tile_rows(blk + 1, off, kvalid[1]);
          issue(s1, off);
        }
        compute(s0, kvalid[0], blk);
        if (blk + 1 >= hi) break;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (blk + 2 < hi) {
          tile_rows(blk + 2, off, kvalid[0]);
          issue(s0, off);
        }
        compute(s1, kvalid[1], blk + 1);
      }
    }
    __syncthreads();   // every wave is done with the stages

    // Row sums over the 4 lanes of a row.
    float l_tot = st.l_lane;
    l_tot += __shfl_xor(l_tot, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    float m_fin = st.m_run;

    const bool final_out = nsplit == 1;
    const int64_t orow_base = final_out ? (int64_t)item * a.M : (int64_t)(slot0 + split) * a.M;

    if constexpr (NT == 1) {
      if (row_ok) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        const int64_t orow = orow_base + row;
        if (final_out) {
          uint16_t* orp = a.o + orow * kDv + 4 * g;
#pragma unroll
          for (int dt = 0; dt < 32; ++dt) {
            bf16x4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = (__bf16)(st.oacc[dt][i] * inv);
            *reinterpret_cast<bf16x4*>(orp + 16 * dt) = v;
          }
        } else {
          float* orp = a.part_o + orow * kDv + 4 * g;
#pragma unroll
          for (int dt = 0; dt < 32; ++dt) *reinterpret_cast<floatx4*>(orp + 16 * dt) = st.oacc[dt] * inv;
        }
        if (g == 0) {
          const float lse = l_tot > 0.f ? m_fin * kLn2 + logf(l_tot) : -INFINITY;
          if (final_out) a.lse[orow] = lse; else a.part_lse[orow] = lse;
        }
      }
    } else {
      // Merge the NT key groups of each row through LDS.
      if (g == 0) {
        red_m[tg][rg * 16 + li] = m_fin;
        red_l[tg][rg * 16 + li] = l_tot;
      }
      __syncthreads();
      float m_all = -INFINITY;
#pragma unroll
      for (int j = 0; j < NT; ++j) m_all = fmaxf(m_all, red_m[j][rg * 16 + li]);
      float l_all = 0.f;
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const float mj = red_m[j][rg * 16 + li];
        l_all += mj == -INFINITY ? 0.f : red_l[j][rg * 16 + li] * fast_exp2(mj - m_all);
      }
      const float f = m_fin == -INFINITY ? 0.f : fast_exp2(m_fin - m_all);
      const float inv = l_all > 0.f ? 1.f / l_all : 0.f;
      // Each wave parks its scaled accumulator: region [tg] = [16 rows][516] fp32.
      constexpr int kStride = 516;
      constexpr int kRegion = 16 * kStride * 4;
      static_assert(2 * kRegion <= kTileBytes, "merge regions must fit the stages");
      char* region = (tg < 2 ? s0 : s1) + (tg & 1) * kRegion;
      float* myreg = reinterpret_cast<float*>(region) + li * kStride + 4 * g;
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) *reinterpret_cast<floatx4*>(myreg + 16 * dt) = st.oacc[dt] * (f * inv);
      __syncthreads();
      // Wave tg sums columns [128 tg, 128 tg + 128): lane -> row lane / 4, 32 columns.
      const int orow_l = lane >> 2;
      const int col0 = 128 * tg + 32 * (lane & 3);
      floatx4 acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const float* rj = reinterpret_cast<const float*>((j < 2 ? s0 : s1) + (j & 1) * kRegion) +
                          orow_l * kStride + col0;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += *reinterpret_cast<const floatx4*>(rj + 4 * e);
      }
      const int r_out = mt * C::kRows + rg * 16 + orow_l;
      if (r_out < a.M) {
        const int64_t orow = orow_base + r_out;
        if (final_out) {
          uint16_t* orp = a.o + orow * kDv + col0;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            bf16x4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = (__bf16)acc[e][i];
            *reinterpret_cast<bf16x4*>(orp + 4 * e) = v;
          }
        } else {
          float* orp = a.part_o + orow * kDv + col0;
#pragma unroll
          for (int e = 0; e < 8; ++e) *reinterpret_cast<floatx4*>(orp + 4 * e) = acc[e];
        }
      }
      if (tg == 0 && g == 0 && row_ok) {
        const float lse = l_all > 0.f ? m_all * kLn2 + logf(l_all) : -INFINITY;
        const int64_t orow = orow_base + row;
        if (final_out) a.lse[orow] = lse; else a.part_lse[orow] = lse;
      }
      __syncthreads();   // regions are reused by the next run's tiles
    }
  }
}

// Merge of the partial results of items split over several workers, and the
// empty result of items with no key.
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a) {
  const int item = blockIdx.x;
  const int slot0 = a.num_splits[item];
  const int n = a.num_splits[item + 1] - slot0;
  if (n == 1) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  typedef __bf16 bf16x8l __attribute__((ext_vector_type(8)));
  for (int r = blockIdx.y * 4 + wave; r < a.M; r += 4 * gridDim.y) {
    const int64_t orow = (int64_t)item * a.M + r;
    float mx = -INFINITY;
    for (int k = 0; k < n; ++k) mx = fmaxf(mx, a.part_lse[(int64_t)(slot0 + k) * a.M + r]);
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    float tot = 0.f;
    if (mx != -INFINITY) {
      for (int k = 0; k < n; ++k) {
        const int64_t prow = (int64_t)(slot0 + k) * a.M + r;
        const float lk = a.part_lse[prow];
        const float wk = lk == -INFINITY ? 0.f : expf(lk - mx);
        tot += wk;
        const floatx4* src = reinterpret_cast<const floatx4*>(a.part_o + prow * kDv + 8 * lane);
        const floatx4 v0 = src[0], v1 = src[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[e] += wk * v0[e];
          acc[4 + e] += wk * v1[e];
        }
      }
    }
    const float inv = tot > 0.f ? 1.f / tot : 0.f;
    bf16x8l v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (__bf16)(acc[e] * inv);
    *reinterpret_cast<bf16x8l*>(a.o + orow * kDv + 8 * lane) = v;
    if (lane == 0) a.lse[orow] = tot > 0.f ? mx + logf(tot) : -INFINITY;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int variant, hipStream_t stream) {
  const int groups = (a.num_workers + 7) / 8;
  if (variant == kVariantRows16) {
    const int grid = a.m_tiles == 1 ? a.num_workers : groups * 8 * a.m_tiles;
    hipLaunchKernelGGL((decode_kernel<1, 4>), dim3(grid), dim3(256), 0, stream, a);
  } else {
    const int grid = a.m_tiles == 1 ? a.num_workers : groups * 8 * a.m_tiles;
    hipLaunchKernelGGL((decode_kernel<4, 1>), dim3(grid), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const DecodeArgs& a, hipStream_t stream) {
  if (a.num_items == 0) return hipSuccess;
  const int gy = min((a.M + 3) / 4, 32);
  hipLaunchKernelGGL(combine_kernel, dim3(a.num_items, gy), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
