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
//    runs of 64-key tiles the scheduler gave it (see mla_plan.hip) as one flat
//    stream of tiles that crosses item boundaries, so the first tile of the
//    next item is already on its way while the current item is finished.
//  * Every 64-row tile (73,728 B) is copied HBM -> LDS with
//    global_load_lds_dwordx4: one instruction moves 8 rows x 128 B, so each
//    wave instruction reads whole 128-byte lines.  Rows are placed in LDS in
//    8-row x 128-B blocks with an XOR swizzle of the 16-byte chunks, which
//    spreads both the row-fragment reads of QK^T and the transposed reads of
//    PV over the LDS banks.  Two stages: tile t + 1 is requested before the
//    wait for tile t.  The copies are issued from inline assembly and waited
//    for with explicit vmcnt counts (see copy_to_lds_16).
//  * S^T = K Q^T on the matrix cores: A = key rows read from LDS, B = query
//    rows held in registers (v_mfma_f32_16x16x32_bf16 for items of up to 16
//    rows, v_mfma_f32_32x32x16_bf16 for larger ones).
//  * Online softmax in base 2 (scores pre-multiplied by scale*log2(e)).  The
//    running reference of a row only moves when the row max exceeds it by more
//    than 8 (a factor 2^8), so the O accumulators are rescaled a few times per
//    run instead of every tile; numerator and denominator share the reference,
//    so the result is the same.
//  * O^T += V^T P^T with the same MFMA; V^T fragments come from LDS through
//    ds_read_b64_tr_b16.  Items of up to 16 query rows (the memory-bound
//    decode case) split each tile's keys over the 4 waves for QK^T and the
//    512 output columns for PV, exchanging P through LDS, so a run ends
//    without merging partial outputs across waves.  Larger items: see the
//    variants below.
//  * Keys past a sequence's length inside its last page, and sparse padding
//    entries, are loaded from a valid row of the same sequence and masked to
//    -inf, so no value outside the key set (e.g. NaN garbage) is ever read.
//  * Runs covering a whole item write bf16 O and fp32 LSE directly; other runs
//    write partials (O normalised by the run's own sum and rounded to bf16,
//    LSE in fp32) that combine_kernel merges (log-sum-exp weights in fp32).
//    Storing the partial O in the output's precision halves the bytes the
//    split runs write and the merge reads; it adds at most one bf16 rounding
//    of the largest partial to the merged value.  In the
//    single-launch mode (FUSED) the last run of an item to finish merges them
//    here instead: partials are stored and loaded at agent scope, which is
//    coherent across the XCDs' L2s without write-back or invalidation, and
//    arrivals are counted with agent-scope atomics once a run's stores are
//    complete (no release/acquire fence, which on this chip writes back and
//    invalidates the whole L2 of the XCD).
#pragma once

#include "mla_common.h"

#include <math.h>

#include <type_traits>
#include <utility>

namespace mla {
namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLazy = 8.f;   // log2 of the growth allowed before a rescale

// XOR pattern of the 16-byte chunks of tile row t (a bijection on t & 7 for
// each parity of t >> 3).  Any 16 consecutive rows then put a given chunk in
// 16 distinct 16-byte bank groups, and so do the 4-row x 2-chunk patterns of
// the transposed reads.
__device__ __forceinline__ int swz(int t) { return (((t & 3) << 1) | ((t >> 2) & 1)) ^ (((t >> 3) & 1) << 1); }
// The rows16 variant's pattern, for its K reads (16 rows, one chunk each per
// quarter wave) and V^T reads (8-byte halves of chunk pairs of 8 rows per
// quarter wave).  Found by measuring SQ_LDS_BANK_CONFLICT for candidate
// patterns on both access shapes: this one leaves both without conflicts.
__device__ __forceinline__ int swz16(int t) { return t & 7; }

// XOR pattern of the 16-byte chunks of row t in a copied FP8 tile, whose
// codes the MFMA operands are read from: the rows of any 16-row group aligned
// to 16 that share a parity get 8 distinct patterns, so that a quarter wave
// reading one chunk of each of 16 rows hits 16 distinct 16-byte bank groups.
__device__ __forceinline__ int raw_swz(int t) { return (t >> 1) & 7; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions over lane pairs (l, l ^ 32) and (l, l ^ 16) with the gfx950 lane
// swaps (v_permlane32_swap / v_permlane16_swap on two copies of the value):
// the first result holds the lower lane's value, the second the upper one's,
// so both lanes of a pair combine the same operands in the same order.
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane i
// receives element i % 4 of the 8-byte words addressed by lanes 4 e + i / 4,
// e = 0..3, i.e. one column of the 4 x 16 block the group points at.
__device__ __forceinline__ bf16x4 read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(p));
}

// Decode variants.  All use 4 waves, 64-key tiles and two LDS stages.
//  Rows16 (items of at most 16 query rows): wave tg computes the scores of
//    keys 16 tg .. 16 tg + 15 (v_mfma_f32_16x16x32_bf16) and, once the
//    probabilities of the whole tile are exchanged through LDS, output columns
//    128 tg .. 128 tg + 127 over all 64 keys.
//  Rows64 (larger items, 64-row tiles): wave = 2 pair + half; the pair owns 32
//    query rows, and the wave computes the scores of keys 32 half .. + 31 and
//    output columns 256 half .. + 255 (v_mfma_f32_32x32x16_bf16), exchanging
//    the probabilities with its partner through LDS.
//  Rows128 (items of more than 64 rows over bf16 caches, 128-row tiles): each
//    wave owns 32 query rows over all 64 keys and all 512 output columns, its
//    32 x 512 fp32 output block in the 256 accumulation registers, so no
//    probability or softmax state crosses waves.
// In all, the waves sharing a row share its softmax reference, so no partial
// outputs are merged when a run ends.
// With packed FP8 rows (KV8) the tiles are copied as they are stored (41 KB
// per 64 rows) into the two stages, and the MFMA operands are read from the
// codes: K fragments by 8-byte reads, V^T fragments by transposed 8-bit reads,
// converted to bf16 in registers (exact: every E4M3 value is a bf16 value).
// The block scales stay out of the bf16 operands, so no dequantized value is
// rounded: QK^T keeps one accumulation per 128-value block and adds them up
// with the keys' scales, and PV takes each key's scale (for the output
// columns' block) into its probability.
template <int V, bool KV8, int D>
struct Cfg {
  static_assert(D == 576 || D == 512, "latent rows of 576 (512 + 64 RoPE) or 512 values");
  static_assert(!KV8 || D == 576, "packed FP8 rows hold 576 values");
  static constexpr bool kWide = V != kVariantRows16;     // 32 rows per wave, 32x32 MFMAs
  static constexpr bool kFull = V == kVariantRows128;    // a wave covers all keys and columns of its rows
  static_assert(!kFull || !KV8, "the 128-row variant reads bf16 rows");
  static constexpr int kCG = D / 64;                     // 128-byte chunk groups of a bf16 row
  static constexpr int kWaves = 4;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kRows = kFull ? 128 : kWide ? 64 : 16;   // query rows per workgroup
  // Copy instructions per wave per tile.  bf16: the wave's 16 rows x 9
  // chunk groups of 128 B.  FP8: its 16 rows x 5 segments of 128 B (latent
  // bytes 0..511, RoPE bytes 528..655), plus four 4-byte copies that put the
  // 16 rows' scales of each block into a [block][row] table.
  static constexpr int kLoads = KV8 ? 14 : 2 * kCG;
  static constexpr int kLaneRows = 2;                    // tile rows each lane copies (8 lanes per row)
  static constexpr int kOffs = KV8 ? 3 : 2;              // copy offsets per lane (FP8: + the scale row)
  static constexpr int kRowB = KV8 ? kRowBytes8 : 2 * D;      // bytes per cached row
  static constexpr int kTileB = kPage * 2 * D;                 // bytes of a tile in the bf16 layout
  static constexpr int kStageBytes = KV8 ? kRaw8Bytes : kTileB;
  static constexpr int kQf = kWide ? D / 16 : D / 32;    // bf16x8 B-operand fragments of Q per lane
  static constexpr int kRowsPerWave = kWide ? 32 : 16;   // rows of the softmax state a wave holds
};

// s_waitcnt operand (gfx9 layout: vmcnt in bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8) that waits until at most n vector-memory operations of the
// wave are outstanding and does not wait on the other counters.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitLds = (15) | (3 << 14) | (7 << 4);   // lgkmcnt(0) only

// Wave-uniform read of one int through the scalar data cache (the tables read
// this way are never written by these kernels).  It is counted by lgkmcnt, so
// waiting for it never waits for the tile copies in flight.
__device__ __forceinline__ int read_scalar(const int32_t* p) {
  int v;
  asm volatile("s_load_dword %0, %1, 0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  return v;
}
// Two such reads in flight together, one wait.
__device__ __forceinline__ void read_scalar2(const int32_t* p0, const int32_t* p1, int& v0, int& v1) {
  asm volatile("s_load_dword %0, %2, 0\n\ts_load_dword %1, %3, 0\n\ts_waitcnt lgkmcnt(0)"
               : "=&s"(v0), "=&s"(v1)
               : "s"(p0), "s"(p1)
               : "memory");
}

// The same for eight consecutive ints (a plan row).
typedef int int32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Eight E4M3 codes (bytes of v, lowest first) as eight bf16 values (exact).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(i32x2 v) {
  bf16x8 r;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)v[k], 1.0f, false);
    const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)v[k], 1.0f, true);
    r[4 * k + 0] = lo[0];
    r[4 * k + 1] = lo[1];
    r[4 * k + 2] = hi[0];
    r[4 * k + 3] = hi[1];
  }
  return r;
}
// Transposed read of 8-bit elements (ds_read_b64_tr_b8).  Within each group
// of 16 lanes, lane i receives as byte b the byte at offset i mod 8 of the
// 8 bytes addressed by lane 2 b + (i >= 8) of the group.
__device__ __forceinline__ i32x2 read_tr8(const char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(p));
}
__device__ __forceinline__ int32x8 read_scalar8(const int32_t* p) {
  int32x8 v;
  asm volatile("s_load_dwordx8 %0, %1, 0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  return v;
}

// One global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane
// l's bytes land at lds + 16 l.  Issued from inline assembly, M0 saved and
// restored around it, so that the compiler does not see an LDS write: it
// would otherwise make every later LDS read wait for all copies in flight,
// which serialises the tile pipeline.  Whoever reads the destination waits
// for the copy with an explicit vmcnt and a barrier.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
__device__ __forceinline__ void copy_to_lds_16(const void* src, unsigned lds) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(src)
      : "memory");
}

// The same copy from a wave-uniform base address (SGPRs) plus a 32-bit
// per-lane offset, and from a 64-bit per-lane address; in both an immediate
// IMM is added to the source address, so a tile's copies share their address
// registers and cost no vector arithmetic.  The instruction adds its
// immediate offset to the LDS address as well (M0 + IMM + 16 lane), so M0
// carries the destination minus IMM (lds >= IMM at every call).
template <int IMM>
__device__ __forceinline__ void copy_to_lds_16_sbase(const char* base, unsigned voff, unsigned lds) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, %3 offset:%4\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds - IMM), "v"(voff), "s"(base), "i"(IMM)
      : "memory");
}
template <int IMM>
__device__ __forceinline__ void copy_to_lds_16_addr(const char* addr, unsigned lds) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, off offset:%3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds - IMM), "v"(addr), "i"(IMM)
      : "memory");
}
// A 64-bit pointer known to be the same in every lane, in scalar registers.
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
}

// f(std::integral_constant<int, i>) for i = 0 .. N - 1, in order (the index is
// a compile-time constant in the body).
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  [&]<int... I>(std::integer_sequence<int, I...>) { (f(std::integral_constant<int, I>{}), ...); }(
      std::make_integer_sequence<int, N>{});
}

// S^T accumulation in VGPRs (the output accumulators fill the AGPRs).  The
// compiler does not see these as MFMAs: a VALU read of the result must wait
// (see mfma_result_wait).
__device__ __forceinline__ void mfma_v(floatx16& acc, bf16x8 a, bf16x8 b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ floatx16 mfma_v0(bf16x8 a, bf16x8 b) {
  floatx16 d;
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  return d;
}
__device__ __forceinline__ void mfma_result_wait() { asm volatile("s_nop 15\n\ts_nop 3" ::: "memory"); }
// This lane's index, produced where it is used by an instruction the
// compiler cannot hoist, so that per-lane LDS addresses built from it are
// remade at each use instead of staying live (and spilled) across a tile loop.
__device__ __forceinline__ int lane_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}
__device__ __forceinline__ float agpr_zero() {
  float r;
  asm volatile("v_accvgpr_write_b32 %0, 0" : "=a"(r));
  return r;
}
__device__ __forceinline__ float agpr_read(float x) {
  float r;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(x));
  return r;
}
// Multiply the accumulators of one wave's O block, held in AGPRs, by alpha:
// each value is moved to a VGPR, multiplied and moved back.  This is the cold
// path of the lazy softmax reference (it runs only when a row maximum grows
// by more than 2^8).  The MFMAs that wrote the block retired long before (a
// whole QK^T chain lies in between); the leading NOPs cover their result
// latency anyway, and the trailing one the VALU write before the next MFMA
// reads the block.
__device__ __forceinline__ void scale_agpr_block(floatx16& acc, float alpha) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float e = acc[i];
    float t;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(e), "=&v"(t)
                 : "v"(alpha));
    acc[i] = e;
  }
  asm volatile("s_nop 4" ::: "memory");
}

// Same for 4 bytes per lane (global_load_lds_dword): lane l's word lands at lds + 4 l.
__device__ __forceinline__ void copy_to_lds_4(const void* src, unsigned lds) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dword %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(src)
      : "memory");
}

// Workgroup barrier that does not wait for the wave's outstanding global
// loads (the copies into the other LDS stage stay in flight across it).  The
// caller has already waited for whatever the barrier must publish; the LDS
// accesses of this wave are completed first, and the memory clobber keeps the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_keep_loads() {
  __builtin_amdgcn_s_waitcnt(kWaitLds);
  asm volatile("s_barrier" ::: "memory");
}

// Partials of split items: O in bf16 (the output's precision), LSE in fp32.
// In the single-launch mode the runs of an item, which may sit on different
// XCDs (each with its own L2, not coherent with the others), exchange them
// through memory: stores and loads at agent scope (sc1), so no L2 write-back
// or invalidate is needed.
//
// Eight bf16 partial values (16 bytes) as floats: v0 = the first four.
template <bool kAgent>
__device__ __forceinline__ void load_part8(const uint16_t* p, floatx4& v0, floatx4& v1) {
  unsigned w[4];
  if constexpr (!kAgent) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    w[0] = u.x;
    w[1] = u.y;
    w[2] = u.z;
    w[3] = u.w;
  } else {
    uint64_t* q = reinterpret_cast<uint64_t*>(const_cast<uint16_t*>(p));
    const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    w[0] = (unsigned)lo;
    w[1] = (unsigned)(lo >> 32);
    w[2] = (unsigned)hi;
    w[3] = (unsigned)(hi >> 32);
  }
  // a bf16 value is the upper half of the float it denotes
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    v0[2 * i] = __uint_as_float(w[i] << 16);
    v0[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    v1[2 * i] = __uint_as_float(w[2 + i] << 16);
    v1[2 * i + 1] = __uint_as_float(w[2 + i] & 0xffff0000u);
  }
}
template <bool kAgent>
__device__ __forceinline__ float load_part1(const float* p) {
  if constexpr (!kAgent) {
    return *p;
  } else {
    unsigned* q = reinterpret_cast<unsigned*>(const_cast<float*>(p));
    return __uint_as_float(__hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  }
}
__device__ __forceinline__ void store_part4_agent(uint16_t* p, bf16x4 v) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), __builtin_bit_cast(uint64_t, v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_part1_agent(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<unsigned*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// o = 0, lse = -inf for row r of an item with no key (one wave, 8 columns per lane).
__device__ __forceinline__ void write_empty_row(const DecodeArgs& a, int item, int r, int lane) {
  const int64_t orow = q_row(a, item, r);
  *reinterpret_cast<uint4*>(a.o + orow * kDv + 8 * lane) = uint4{0, 0, 0, 0};
  if (lane == 0) a.lse[orow] = -INFINITY;
}

// Log-sum-exp merge of n <= N partials of row r of an item (one wave, 8
// columns per lane): all N reads go out together, unconditionally (reads past
// the n-th repeat the last partial and are not used), so the merge waits for
// one memory latency; then the arithmetic.
template <int N, bool kAgent>
__device__ __forceinline__ void merge_row_small(const DecodeArgs& a, int64_t orow, int slot0, int n, int r,
                                                int lane) {
  float lk[N];
  floatx4 v0[N], v1[N];
  const int64_t stride = (int64_t)a.part_rows * kDv;
  const uint16_t* o_col = a.part_o + ((int64_t)slot0 * a.part_rows + r) * kDv + 8 * lane;
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const int kk = k < n ? k : n - 1;
    lk[k] = load_part1<kAgent>(a.part_lse + (int64_t)(slot0 + kk) * a.part_rows + r);
    load_part8<kAgent>(o_col + kk * stride, v0[k], v1[k]);
  }
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < N; ++k)
    if (k < n) mx = fmaxf(mx, lk[k]);
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  float tot = 0.f;
  if (mx != -INFINITY) {
#pragma unroll
    for (int k = 0; k < N; ++k) {
      if (k < n) {
        const float wk = lk[k] == -INFINITY ? 0.f : expf(lk[k] - mx);
        tot += wk;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[i] += wk * v0[k][i];
          acc[4 + i] += wk * v1[k][i];
        }
      }
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (__bf16)(acc[i] * inv);
  *reinterpret_cast<bf16x8*>(a.o + orow * kDv + 8 * lane) = v;
  if (lane == 0) a.lse[orow] = tot > 0.f ? mx + logf(tot) : -INFINITY;
}

// Log-sum-exp merge of the n >= 1 partials of row r of an item, one wave per
// row, 8 columns per lane.  Up to 8 partials: one batch of reads (sized 2, 4
// or 8).  More: the partial LSEs are read lane-parallel for the max, and the
// weighted sum of the partial rows keeps 4 reads in flight.
template <bool kAgent>
__device__ __forceinline__ void merge_row(const DecodeArgs& a, int item, int slot0, int n, int r, int lane) {
  const int64_t orow = q_row(a, item, r);
  if (n <= 2) return merge_row_small<2, kAgent>(a, orow, slot0, n, r, lane);
  if (n <= 4) return merge_row_small<4, kAgent>(a, orow, slot0, n, r, lane);
  if (n <= 8) return merge_row_small<8, kAgent>(a, orow, slot0, n, r, lane);
  float mx = -INFINITY;
  for (int k = lane; k < n; k += 64)
    mx = fmaxf(mx, load_part1<kAgent>(a.part_lse + (int64_t)(slot0 + k) * a.part_rows + r));
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) mx = fmaxf(mx, __shfl_xor(mx, d, 64));
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  float tot = 0.f;
  if (mx != -INFINITY) {
    const float* lse_col = a.part_lse + (int64_t)slot0 * a.part_rows + r;
    const uint16_t* o_col = a.part_o + ((int64_t)slot0 * a.part_rows + r) * kDv + 8 * lane;
    const int64_t stride = (int64_t)a.part_rows * kDv;
#pragma unroll 4
    for (int k = 0; k < n; ++k) {
      const float lk = load_part1<kAgent>(lse_col + (int64_t)k * a.part_rows);
      const float wk = lk == -INFINITY ? 0.f : expf(lk - mx);
      tot += wk;
      floatx4 v0, v1;
      load_part8<kAgent>(o_col + k * stride, v0, v1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] += wk * v0[i];
        acc[4 + i] += wk * v1[i];
      }
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (__bf16)(acc[i] * inv);
  *reinterpret_cast<bf16x8*>(a.o + orow * kDv + 8 * lane) = v;
  if (lane == 0) a.lse[orow] = tot > 0.f ? mx + logf(tot) : -INFINITY;
}

template <int V, bool SPARSE, bool KV8, int D, bool FUSED>
__global__ __launch_bounds__(256, 1) void decode_kernel(DecodeArgs a) {
  using C = Cfg<V, KV8, D>;
  constexpr bool kWide = C::kWide;
  constexpr bool kFull = C::kFull;
  constexpr int kRw = C::kRowsPerWave;
  // vector-memory operations issued per wave for a tile: copy, sparse index loads
  constexpr int kRaw = C::kOffs;
  constexpr int kWaitKeepCopy = waitcnt_vm(C::kLoads);
  constexpr int kWaitKeepRawCopy = waitcnt_vm(C::kLoads + kRaw);
  static_assert(C::kLoads + kRaw < 64, "vmcnt holds 6 bits");
  static_assert(C::kLoads + 2 * C::kCG + kRaw < 64, "vmcnt holds 6 bits (with a query-row copy)");
  __shared__ __attribute__((aligned(1024))) char s0[C::kStageBytes];
  __shared__ __attribute__((aligned(1024))) char s1[C::kStageBytes];
  __shared__ __attribute__((aligned(16))) unsigned char kvalid[4][64];   // sparse key validity, tile t -> t & 3
  // per-wave row maxima of the tile and row sums at the end of a run (the
  // 128-row variant keeps every row inside one wave and needs neither)
  __shared__ float red_m[kFull ? 1 : 4][kFull ? 1 : kRw];
  __shared__ float red_l[kFull ? 1 : 4][kFull ? 1 : kRw];
  __shared__ int red_need[4];         // wide: wave wants the softmax reference moved
  // Probabilities of the tile in bf16.  Rows16: P^T [row][key pair block c][lane
  // group g][8], slot 4 h + i of (c, g) = key 16 (2 c + h) + 4 g + i.  Wide: the
  // B operands of the wave's two PV k-steps, [wave][k-step][lane][8].
  // rows16: bytes per row of the probability buffer, padded by 8 so that its
  // 16-byte reads and 8-byte writes hit no bank conflict (measured; 128 and
  // 144 do)
  constexpr int kPRow = 136;
  __shared__ __attribute__((aligned(16))) char pbuf[kFull ? 16 : kWide ? 4 * 2 * 64 * 16 : 16 * kPRow];
  const float* sc_tab = nullptr;   // FP8: scale table [block][row] of the tile being computed
  // Wide: index data of the next tiles (sparse: the 64 index-list entries;
  // dense: the page id, in every entry), copied in by wave 0 ([tile & 3][64])
  // a step ahead, so that neither a register load left behind a tile copy nor
  // a scalar round trip sits on the critical path of a step (the step's wait
  // and barrier make it visible to every wave).
  __shared__ __attribute__((aligned(256))) int idxbuf[kWide ? 4 : 1][64];
  // Wide, sparse: the block-table entries (pages) of the rows of a tile,
  // loaded one step ahead ([tile & 1][wave][lane]: lane l of wave w holds the
  // page of row 16 w + l % 16).
  __shared__ __attribute__((aligned(256))) int pgbuf[(kWide && SPARSE) ? 2 : 1][4][64];
  // Rows16, FP8 (whose copied tiles leave room): the query rows of the item a
  // tile starts, copied in by wave 0 with that tile, in the tile layout.  Two
  // slots, since an item of one tile can start and end between two reads.
  constexpr bool kQSlots = KV8 && !kWide;
  __shared__ __attribute__((aligned(1024))) char qbuf[kQSlots ? 2 : 1][kQSlots ? 16 * 2 * D : 16];

  // The arguments on the way to the first tile copy, loaded in one go (left
  // to itself, the compiler loads each one where it is first used, a round
  // trip apiece).
  asm volatile("" ::"s"(a.q), "s"(a.kv), "s"(a.block_table), "s"(a.seqlens), "s"(a.plan), "s"(a.m_tiles),
               "s"(a.num_workers), "s"(a.max_blocks), "s"(a.s_q), "s"(a.M), "s"(a.h_kv), "s"(a.G),
               "s"(a.topk));

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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int g = lane >> 4;      // lane group of 16
  const int li = lane & 15;
  // rows16: the wave's key group / column quarter.  64-row variant: pair and
  // half.  128-row variant: the wave's 32 rows, all keys and columns (half 0).
  const int tg = wave;
  const int pair = kFull ? wave : wave >> 1, half = kFull ? 0 : wave & 1;
  const int lrow = kWide ? (lane & 31) : li;   // row of the lane inside its wave's rows
  const int hl = lane >> 5;                    // wide: k half of the lane's MFMA operands
  const int row0 = mt * C::kRows;
  const int row = row0 + (kWide ? 32 * pair : 0) + lrow;   // query row inside the item (S^T column)
  const bool row_ok = row < a.M;
  constexpr bool sparse = SPARSE;      // top-k index lists (a.topk > 0)
  // chunk swizzle of a bf16 tile row (the variants read their tiles differently)
  auto tswz = [](int t) __attribute__((always_inline)) { return kWide ? swz(t) : swz16(t); };

  const int32x8 prow = read_scalar8(a.plan + kPlanWords * (1 + w));
  const int it_first = prow[0], blk_first = prow[1], it_last = prow[2], blk_end = prow[3],
            split_first = prow[4];

  if (it_first >= 0) {
    // LDS read offsets of this lane.  Byte offset of chunk c of tile row t:
    // ((t / 8) * kCG + c / 8) * 1024 + (t % 8) * 128 + ((c % 8) ^ tswz(t)) * 16
    // (kCG = 9 chunk groups of 128 B for 576-value rows, 8 for 512).
    int k_base, v_base;
    int k_x[4];       // rows16: [0] even ks, [1] odd ks; wide: by ks & 3
    int v_x[2][4];    // rows16: [0][dt & 3]; wide: [second 4 keys][db & 1]
    if constexpr (!kWide) {
      //  K: key row t = 16 tg + li, chunk 4 ks + g.
      const int tk = 16 * tg + li;
      k_base = ((tk >> 3) * C::kCG << 10) + ((tk & 7) << 7);
      k_x[0] = ((g ^ tswz(tk)) << 4);
      k_x[1] = (((4 + g) ^ tswz(tk)) << 4);
      //  V^T: source row t = 16 s + 4 g + li / 4 of key subtile s, columns
      //  128 tg + 16 dt + 4 (li & 3) .. + 3: chunk 16 tg + 2 dt + (li & 3) / 2, half li & 1.
      const int tv = 4 * g + (li >> 2);
      v_base = ((tv >> 3) * C::kCG << 10) + ((tv & 7) << 7) + ((li & 1) << 3) + ((2 * tg) << 10);
#pragma unroll
      for (int d = 0; d < 4; ++d) v_x[0][d] = (((2 * d + ((li & 3) >> 1)) ^ tswz(tv)) << 4);
    } else {
      //  K: key row t = 32 half + lrow, chunk 2 ks + hl.
      const int tk = 32 * half + lrow;
      k_base = ((tk >> 3) * C::kCG << 10) + ((tk & 7) << 7);
#pragma unroll
      for (int b = 0; b < 4; ++b) k_x[b] = (((2 * b + hl) ^ swz(tk)) << 4);
      //  V^T for PV k-step j (keys 16 j .. 16 j + 15 in the order of the score
      //  accumulators) and column block db: source rows 16 j + 4 hl + li / 4
      //  (+ 8 for the second read), columns 256 half + 32 db + 16 (g & 1) +
      //  4 (li & 3) .. + 3: chunk 32 half + 4 db + 2 (g & 1) + (li & 3) / 2.
      const int tv = 4 * hl + (li >> 2);
      v_base = (tv << 7) + ((li & 1) << 3) + ((4 * half) << 10);
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          v_x[e][b] = (((4 * b + 2 * (g & 1) + ((li & 3) >> 1)) ^ swz(tv + 8 * e)) << 4);
    }

    // Rows16 FP8: the MFMA operands come straight from the copied tile, the
    // codes converted in registers.  K (QK^T): row t = 16 tg + li; latent
    // k-steps 2 p and 2 p + 1 take values 64 p + 16 g .. + 15 (one 16-byte
    // chunk of segment p / 2; the query fragments follow the same order), the
    // RoPE k-steps 16, 17 the bf16 chunk 4 (ks - 16) + g of segment 4.  V^T
    // (PV): for a transposed read this lane addresses row 32 c + 8 G + b,
    // bytes 16 dt + 8 h .. + 7 of latent segment tg (G = lane / 16,
    // b = (lane % 16) / 2, h = lane % 2), which hands lane i of each 16-lane
    // group column 16 dt + i of the 8 rows 32 c + 8 G + 0..7.
    int k8_base = 0, v8_base = 0, v8_sw = 0, k8_sw = 0;
    int k8_x[4] = {0, 0, 0, 0}, r8_x[2] = {0, 0}, v8_x[4] = {0, 0, 0, 0};
    if constexpr (kWide && KV8) {
      // Wide FP8: K row tk = 32 half + lrow; latent k-steps 2 p and 2 p + 1
      // take values 32 p + 16 hl .. + 15 (chunk 2 (p % 4) + hl of segment
      // p / 4), the RoPE k-steps 32..35 the bf16 chunk 2 (ks - 32) + hl of
      // segment 4.  V^T for
      // PV k-step j and column block db: this lane addresses row
      // 16 j + 8 (G / 2) + b, bytes 32 (db % 4) + 16 (G % 2) + 8 h .. + 7 of
      // latent segment 2 half + db / 4, which hands lane i of each 16-lane
      // group column 256 half + 32 db + 16 (G % 2) + i of the 8 rows
      // 16 j + 8 (G / 2) + 0..7: the A operand of a 32x32x16 MFMA.
      const int tk = 32 * half + lrow;
      k8_sw = raw_swz(tk);
      k8_base = ((tk >> 3) * 5 << 10) + ((tk & 7) << 7);
      const int G = lane >> 4, b = (lane & 15) >> 1, h = lane & 1;
      v8_base = ((((G >> 1) * 5) + 2 * half) << 10) + (b << 7) + 8 * h;
      v8_sw = raw_swz(8 * (G >> 1) + b);
#pragma unroll
      for (int q = 0; q < 4; ++q) v8_x[q] = ((2 * q + (G & 1)) ^ v8_sw) << 4;   // PV chunk offsets by db % 4
    }
    if constexpr (!kWide && KV8) {
      const int tk = 16 * tg + li, sw = raw_swz(tk);
      k8_base = ((tk >> 3) * 5 << 10) + ((tk & 7) << 7);
#pragma unroll
      for (int q = 0; q < 2; ++q) k8_x[q] = ((4 * q + g) ^ sw) << 4;
#pragma unroll
      for (int e = 0; e < 2; ++e) r8_x[e] = (4 << 10) + (((4 * e + g) ^ sw) << 4);
      const int G = lane >> 4, b = (lane & 15) >> 1, h = lane & 1;
      v8_base = ((G * 5 + tg) << 10) + (b << 7) + 8 * h;
      v8_sw = raw_swz(8 * G + b);   // that of row 32 c + 8 G + b
    }

    // Tile rows this lane copies: t = 8 * (2 wave + r) + lane / 8 (the wave's 16 rows).
    int cp_row[C::kLaneRows];
    int cp_swz[C::kLaneRows];
#pragma unroll
    for (int r = 0; r < C::kLaneRows; ++r) {
      cp_row[r] = 8 * (2 * wave + r) + (lane >> 3);
      cp_swz[r] = tswz(cp_row[r]);
    }
    const char* kv_bytes = reinterpret_cast<const char*>(a.kv);

    // Sequence length of each of this worker's items, lane j holding item
    // it_first + j, and the split-slot prefix at item it_first + j (read in
    // the prologue, before any copy is in flight: the end of an item then
    // waits for no load).
    int lens_v = 0, splits_v = 0;
    if (lane <= it_last - it_first) {
      const int x = it_first + lane;
      lens_v = a.seqlens[item_seq(a, x)];
    }
    if (lane <= it_last - it_first + 1) splits_v = a.num_splits[it_first + lane];
    // The first item's length and the page of the first tile (dense) come in
    // by scalar loads in the prologue, so that the first copy does not wait
    // for the vector loads (the other lengths, the query rows).
    int len_first = 0, page_first = 0;
    auto item_len = [&](int x) __attribute__((always_inline)) -> int {      // x is wave-uniform
      const int j = x - it_first;
      if (j == 0) return len_first;
      if (j < 64) return __builtin_amdgcn_readlane(lens_v, j);
      return read_scalar(a.seqlens + item_seq(a, x));
    };
    auto seg_hi = [&](int x) __attribute__((always_inline)) -> int {         // end block of this worker's run in item x
      if (x == it_last) return blk_end;
      if constexpr (sparse) return a.nb_sparse;
      const int len = item_len(x);
      return len > 0 ? (len + kPage - 1) / kPage : 0;
    };
    // Sparse tile blk of an item: its index list (main, or the auxiliary
    // cache's after the main list's nb1 tiles), that list's length, and the
    // tile's first entry.
    struct SparseList {
      const int32_t* list;
      int n, e0;
      bool aux;
    };
    auto sparse_list = [&](int item, int blk) __attribute__((always_inline)) -> SparseList {
      const int64_t tok = div_by(item, (unsigned)a.h_kv, a.head_mul);
      if (blk < a.nb1) return {a.indices + tok * a.topk, a.topk, blk * kPage, false};
      return {a.indices2 + tok * a.topk2, a.topk2, (blk - a.nb1) * kPage, true};
    };
    // Tile after (item, blk) in this worker's runs (hi = end block of the run
    // in `item`); ni = -1 at the end.
    auto advance = [&](int item, int blk, int hi, int& ni, int& nb, int& nhi) __attribute__((always_inline)) {
      if (blk + 1 < hi) {
        ni = item;
        nb = blk + 1;
        nhi = hi;
        return;
      }
      for (int x = item + 1; x <= it_last; ++x) {
        const int h = seg_hi(x);
        if (h > 0) {
          ni = x;
          nb = 0;
          nhi = h;
          return;
        }
      }
      ni = -1;
      nb = 0;
      nhi = 0;
    };

    // Copy addresses of a tile are found in two steps so that the index loads
    // can be issued a whole tile ahead: tile_fetch loads the raw index data
    // (dense: the tile's page id; sparse: this lane's index-list entries),
    // tile_finish turns it into byte offsets (in the cache) of the rows this
    // lane copies, and the sparse key validity of the tile.
    struct TileRaw {
      int v[C::kOffs];
    };
    // FP8: the row whose scales this lane copies (lanes 0..15 of the wave)
    const int sc_row = 16 * wave + (lane & 15);
    // Dense: bytes per page (all heads), and the offsets inside a page of the
    // rows this lane copies (tile_finish adds the page's offset).
    const int64_t page_bytes = (int64_t)kPage * a.h_kv * C::kRowB;
    int64_t row_in_page[C::kOffs];
#pragma unroll
    for (int r = 0; r < C::kOffs; ++r)
      row_in_page[r] = (int64_t)(KV8 && r == 2 ? sc_row : cp_row[r < C::kLaneRows ? r : 0]) * a.h_kv * C::kRowB;
    // bf16: the 16-byte chunk this lane copies of each of its rows (the XOR
    // swizzle of the destination row), as a byte offset inside the row's
    // 128-byte chunk groups
    unsigned chunk_off[C::kLaneRows];
#pragma unroll
    for (int r = 0; r < C::kLaneRows; ++r) chunk_off[r] = ((lane & 7) ^ cp_swz[r]) << 4;

    // Where this lane's copies of a tile read from.  Packed FP8 tiles: byte
    // offsets from kv of the rows (off).  bf16 tiles: a dense tile is one
    // page, so its copies read from a base address shared by the wave (the
    // page and latent head) plus a per-lane offset (row and chunk) that is
    // the same for every full tile; a sparse tile's rows are scattered, so
    // each lane keeps the address of its chunk of each row.  Either way the
    // 128-byte chunk group of a copy is an immediate offset.
    struct Src {
      int64_t off[C::kOffs];
      const char* base;
      unsigned voff[C::kLaneRows];
      const char* addr[C::kLaneRows];
    };
    unsigned voff_full[C::kLaneRows];
#pragma unroll
    for (int r = 0; r < C::kLaneRows; ++r) voff_full[r] = (unsigned)row_in_page[r] + chunk_off[r];
    // Indexing probe: the cache offset of every row the copies of tile (item,
    // blk) read, from the same registers the copies use.
    auto record = [&](int item, int blk, const Src& src) __attribute__((always_inline)) {
      if (a.dbg_rows == nullptr) return;
      int64_t* rec = a.dbg_rows + ((int64_t)item * a.dbg_tiles + blk) * kPage;
      if ((lane & 7) == 0) {
#pragma unroll
        for (int r = 0; r < C::kLaneRows; ++r) {
          int64_t o;
          if constexpr (KV8) o = src.off[r];
          else if constexpr (sparse) o = (src.addr[r] - kv_bytes) - chunk_off[r];
          else o = (src.base - kv_bytes) + src.voff[r] - chunk_off[r];
          rec[cp_row[r]] = o;
        }
      }
      if constexpr (KV8) {
        if (lane < 16) rec[a.dbg_plane + sc_row] = src.off[2];
      }
    };
    // bf16 sparse tiles: addresses from the row offsets
    auto seal_sparse = [&](Src& src) __attribute__((always_inline)) {
      if constexpr (!KV8) {
#pragma unroll
        for (int r = 0; r < C::kLaneRows; ++r) src.addr[r] = kv_bytes + src.off[r] + chunk_off[r];
      }
    };
    auto tile_fetch = [&](int item, int blk, TileRaw& raw) __attribute__((always_inline)) {
      if constexpr (!sparse) {
        raw.v[0] = read_scalar(a.block_table + (int64_t)item_seq(a, item) * a.max_blocks + blk);   // not a vector load
      } else {
        const SparseList sl = sparse_list(item, blk);
#pragma unroll
        for (int r = 0; r < C::kLaneRows; ++r) {
          const int e = sl.e0 + cp_row[r];
          raw.v[r] = e < sl.n ? sl.list[e] : -1;
        }
        if constexpr (KV8) {
          const int e = sl.e0 + sc_row;
          raw.v[2] = e < sl.n ? sl.list[e] : -1;
        }
      }
    };
    // Sparse: the rows of a tile in two steps.  translate reads the block
    // table (page of each index-list entry this lane copies; padding reads the
    // sequence's first row, page 0 of the pool if it has none) and records the
    // tile's key validity; finish_pre turns the pages into byte offsets
    // (auxiliary-cache rows taken from the main cache's base).  The wide
    // variant translates a tile one step before it issues its copy, so the
    // block-table loads are complete by then.
    struct TilePre {
      int page[C::kOffs];
      int slot[C::kOffs];
      bool aux;
    };
    auto translate = [&](int item, int blk, const TileRaw& raw, TilePre& pre,
                         unsigned char* vslot) __attribute__((always_inline)) {
      const bool aux = blk >= a.nb1;
      const int b = item_seq(a, item);
      const int32_t* bt_row = aux ? a.block_table2 + (int64_t)b * a.max_blocks2
                                  : a.block_table + (int64_t)b * a.max_blocks;
      const int Ls = aux ? read_scalar(a.seqlens2 + b) : item_len(item);
      pre.aux = aux;
#pragma unroll
      for (int r = 0; r < C::kOffs; ++r) {
        const int idx = raw.v[r];
        const bool ok = sparse_key_valid(idx, Ls);
        const int pos = ok ? idx : 0;
        // the load is unconditional (entry 0 is always inside the table) and
        // its value is not touched here, so nothing waits for it before the
        // next step; slot -1 marks "the pool's first row"
        pre.page[r] = bt_row[pos >> 6];
        pre.slot[r] = (ok || Ls > 0) ? (pos & (kPage - 1)) : -1;
        if (r < C::kLaneRows && (lane & 7) == 0) vslot[cp_row[r]] = ok ? 1 : 0;
      }
    };
    auto finish_pre = [&](int item, const TilePre& pre, Src& src) __attribute__((always_inline)) {
      const int kvh = item - div_by(item, (unsigned)a.h_kv, a.head_mul) * a.h_kv;
      const int64_t base = pre.aux ? (int64_t)(reinterpret_cast<const char*>(a.kv2) - kv_bytes) : 0;
#pragma unroll
      for (int r = 0; r < C::kOffs; ++r) {
        const int64_t crow = pre.slot[r] < 0 ? 0 : (int64_t)pre.page[r] * kPage + pre.slot[r];
        src.off[r] = base + (crow * a.h_kv + kvh) * (int64_t)C::kRowB;
      }
      seal_sparse(src);
    };
    auto tile_finish = [&](int item, int blk, const TileRaw& raw, Src& src,
                           unsigned char* vslot) __attribute__((always_inline)) {
      if constexpr (!sparse) {
        const int L = item_len(item);
        const int kvh = item - div_by(item, (unsigned)a.h_kv, a.head_mul) * a.h_kv;   // latent KV head of the item
        // byte offset of the tile's page and head (wave-uniform), plus each
        // copied row's offset inside the page (precomputed for full tiles;
        // keys past the length read the last valid row)
        const int64_t base = (int64_t)__builtin_amdgcn_readfirstlane(raw.v[0]) * page_bytes +
                             (int64_t)kvh * C::kRowB;
        const int nvalid = min(kPage, L - blk * kPage);
        if constexpr (KV8) {
          if (nvalid == kPage) {
#pragma unroll
            for (int r = 0; r < C::kOffs; ++r) src.off[r] = base + row_in_page[r];
          } else {
#pragma unroll
            for (int r = 0; r < C::kLaneRows; ++r)
              src.off[r] = base + (int64_t)min(cp_row[r], nvalid - 1) * a.h_kv * C::kRowB;
            src.off[2] = base + (int64_t)min(sc_row, nvalid - 1) * a.h_kv * C::kRowB;
          }
        } else {
          src.base = uniform_ptr(kv_bytes + base);
          if (nvalid == kPage) {
#pragma unroll
            for (int r = 0; r < C::kLaneRows; ++r) src.voff[r] = voff_full[r];
          } else {
#pragma unroll
            for (int r = 0; r < C::kLaneRows; ++r)
              src.voff[r] = (unsigned)(min(cp_row[r], nvalid - 1) * a.h_kv * C::kRowB) + chunk_off[r];
          }
        }
      } else {
        TilePre pre;
        translate(item, blk, raw, pre, vslot);
        finish_pre(item, pre, src);
      }
      record(item, blk, src);
    };
    // Copy instruction J (0 .. kLoads - 1, a compile-time constant) of this
    // wave for a tile: 8 rows x 128 B.  bf16 stage layout: chunk group cl of
    // rows 8 (2 wave + r) .. + 7 at ((2 wave + r) * kCG + cl) * 1024.  FP8
    // stage layout: segment sg (0..3: latent bytes 128 sg .., 4: RoPE) of row
    // t at ((t / 8) * 5 + sg) * 1024 + (t % 8) * 128, its 16-byte chunks
    // XOR-swizzled by raw_swz; scale b of row t at kRaw8ScaleOff + 4 (64 b + t).
    auto issue_one = [&](char* stage, const Src& src, auto jc) __attribute__((always_inline)) {
      constexpr int j = decltype(jc)::value;
      if constexpr (!KV8) {
        constexpr int r = j / C::kCG, cl = j % C::kCG;
        const unsigned lds = lds_addr(stage + (wave * C::kLoads + j) * 1024);
        if constexpr (sparse) copy_to_lds_16_addr<cl * 128>(src.addr[r], lds);
        else copy_to_lds_16_sbase<cl * 128>(src.base, src.voff[r], lds);
      } else if constexpr (j < 10) {
        constexpr int r = j / 5, sg = j % 5;
        const char* p = kv_bytes + src.off[r] + (sg < 4 ? sg * 128 : 528) +
                        (((lane & 7) ^ raw_swz(cp_row[r])) << 4);
        copy_to_lds_16(p, lds_addr(stage + ((2 * wave + r) * 5 + sg) * 1024));
      } else {
        constexpr int b = j - 10;
        if (lane < 16)
          copy_to_lds_4(kv_bytes + src.off[2] + 512 + 4 * b, lds_addr(stage + kRaw8ScaleOff + 256 * b + 64 * wave));
      }
    };
    auto issue = [&](char* stage, const Src& src) __attribute__((always_inline)) {
      static_for<C::kLoads>([&](auto jc) __attribute__((always_inline)) { issue_one(stage, src, jc); });
    };
    // Wide: copy the index data of tile (item, blk) into ring slot `slot`.
    // Sparse: its 64 index-list entries (entries past topk repeat the last one;
    // they are padding).  Dense: its page id.
    auto idx_dma = [&](int item, int blk, int slot) __attribute__((always_inline)) {
      const int32_t* src;
      if constexpr (sparse) {
        const SparseList sl = sparse_list(item, blk);
        src = sl.list + min(sl.e0 + lane, sl.n - 1);
      } else {
        src = a.block_table + (int64_t)item_seq(a, item) * a.max_blocks + blk;
      }
      if (wave == 0) copy_to_lds_4(src, lds_addr(&idxbuf[slot & 3][0]));
    };
    auto idx_from_lds = [&](int item, int blk, int slot, TileRaw& raw) __attribute__((always_inline)) {
      if constexpr (sparse) {
        const SparseList sl = sparse_list(item, blk);
#pragma unroll
        for (int r = 0; r < C::kLaneRows; ++r)
          raw.v[r] = sl.e0 + cp_row[r] < sl.n ? idxbuf[slot & 3][cp_row[r]] : -1;
        if constexpr (KV8) raw.v[2] = sl.e0 + sc_row < sl.n ? idxbuf[slot & 3][sc_row] : -1;
      } else {
        raw.v[0] = idxbuf[slot & 3][0];
      }
    };

    // Wide, sparse: the translation of a tile's index entries into rows,
    // split over two steps without registers carried between them (a load
    // result carried across the loop would have the compiler wait for every
    // copy in flight).  translate_lds copies the page of each row's entry
    // (row 16 wave + lane % 16; padding takes entry 0 of the block table) into
    // pgbuf and records the rows' validity; finish_lds, a step later, turns
    // the entries and pages into byte offsets.
    auto sparse_rows = [&](int item, int blk, const int32_t*& bt_row, int& Ls, int64_t& base) __attribute__((always_inline)) {
      const bool aux = blk >= a.nb1;
      const int b = item_seq(a, item);
      bt_row = aux ? a.block_table2 + (int64_t)b * a.max_blocks2 : a.block_table + (int64_t)b * a.max_blocks;
      Ls = aux ? read_scalar(a.seqlens2 + b) : item_len(item);
      base = aux ? (int64_t)(reinterpret_cast<const char*>(a.kv2) - kv_bytes) : 0;
    };
    // Each of the two is split in an LDS read (…_read) and the work on its
    // result (…_use), so that the 128-row variant can issue the read a few
    // MFMAs before the result is needed.
    auto translate_read = [&](int item, int blk, int slot) __attribute__((always_inline)) -> int {
      const SparseList sl = sparse_list(item, blk);
      const int rr = 16 * wave + (lane_here() & 15);
      return sl.e0 + rr < sl.n ? idxbuf[slot & 3][rr] : -1;
    };
    auto translate_use = [&](int item, int blk, int slot, int idx, unsigned char* vslot) __attribute__((always_inline)) {
      const int32_t* bt_row;
      int Ls;
      int64_t base;
      sparse_rows(item, blk, bt_row, Ls, base);
      const bool ok = sparse_key_valid(idx, Ls);
      copy_to_lds_4(bt_row + ((ok ? idx : 0) >> 6), lds_addr(&pgbuf[slot & 1][wave][0]));
      if (lane < 16) vslot[16 * wave + (lane_here() & 15)] = ok ? 1 : 0;
    };
    auto translate_lds = [&](int item, int blk, int slot, unsigned char* vslot) __attribute__((always_inline)) {
      if constexpr (kWide && sparse) translate_use(item, blk, slot, translate_read(item, blk, slot), vslot);
    };
    // The index entries and pages of this lane's rows of a tile.
    struct RowsRaw {
      int idx[C::kOffs];
      int page[C::kOffs];
    };
    auto finish_read = [&](int item, int blk, int slot, RowsRaw& rr) __attribute__((always_inline)) {
      const SparseList sl = sparse_list(item, blk);
#pragma unroll
      for (int r = 0; r < C::kOffs; ++r) {
        const int row = r < C::kLaneRows ? 8 * (2 * wave + r) + (lane_here() >> 3) : sc_row;
        rr.idx[r] = sl.e0 + row < sl.n ? idxbuf[slot & 3][row] : -1;
        rr.page[r] = pgbuf[slot & 1][row >> 4][row & 15];
      }
    };
    auto finish_use = [&](int item, int blk, const RowsRaw& rr, Src& src) __attribute__((always_inline)) {
      const int32_t* bt_row;
      int Ls;
      int64_t base;
      sparse_rows(item, blk, bt_row, Ls, base);
      const int kvh = item - div_by(item, (unsigned)a.h_kv, a.head_mul) * a.h_kv;
#pragma unroll
      for (int r = 0; r < C::kOffs; ++r) {
        const bool ok = sparse_key_valid(rr.idx[r], Ls);
        // padding reads the sequence's first row (the pool's first if it has none)
        const int64_t crow =
            (ok || Ls > 0) ? (int64_t)rr.page[r] * kPage + ((ok ? rr.idx[r] : 0) & (kPage - 1)) : 0;
        src.off[r] = base + (crow * a.h_kv + kvh) * (int64_t)C::kRowB;
      }
      seal_sparse(src);
      record(item, blk, src);
    };
    auto finish_lds = [&](int item, int blk, int slot, Src& src) __attribute__((always_inline)) {
      if constexpr (kWide && sparse) {
        RowsRaw rr;
        finish_read(item, blk, slot, rr);
        finish_use(item, blk, rr, src);
      }
    };

    Src off;   // where this lane's copies of the next tile issued read from

    // Sparse: a tile without a single valid key adds nothing, but its rows
    // need not hold finite values (a sequence with no row at all in a cache
    // has its padding read the pool's first row), and 0 * NaN would reach O
    // through PV.  Such a tile is cleared before it is computed (the test is
    // the same in every wave).
    // Whether a sparse tile has a valid key, and whether all of its keys are
    // (wave-uniform; the 64 keys of the tile are the 64 lanes).
    auto tile_validity = [&](const unsigned char* vslot, bool& any, bool& all) __attribute__((always_inline)) {
      const bool v = vslot[lane] != 0;
      any = __builtin_amdgcn_ballot_w64(v) != 0;
      all = __builtin_amdgcn_ballot_w64(!v) == 0;
    };
    auto clear_if_empty = [&](char* tile, bool any_valid) __attribute__((always_inline)) {
      if constexpr (sparse) {
        if (!any_valid) {
          // the bf16 tile, or (FP8) the copied codes and RoPE values
          constexpr int kClearB = KV8 ? kRaw8ScaleOff : C::kTileB;
          for (int i = threadIdx.x; i < kClearB / 16; i += C::kThreads)
            reinterpret_cast<uint4*>(tile)[i] = uint4{0, 0, 0, 0};
          if constexpr (KV8) reinterpret_cast<float*>(const_cast<float*>(sc_tab))[threadIdx.x] = 0.f;
          barrier_keep_loads();
        }
      }
    };

    // Per-run state of this wave.
    using Acc = typename std::conditional<kWide, floatx16, floatx4>::type;
    bf16x8 qf[C::kQf];    // B operand of S^T, 8 values of row `row` per fragment
    constexpr int kOBlocks = kFull ? 16 : 8;
    Acc oacc[kOBlocks];   // O^T of the wave's output columns, scaled by 2^-m_ref
    float m_ref = -INFINITY;   // softmax reference of row `row` (shared by the waves holding it)
    float l_lane = 0.f;   // sum over this lane's keys of 2^(x - m_ref)

    // Rows past M borrow row 0's values (their scores are masked to -inf), so
    // no select on the loaded data forces an early wait on the loads.
    // Query row of (item, row) = item part (the same in every lane) + row
    // part: dense, row = s G + j of item (b, g) is row (b s_q + s) h_q + g G + j
    // of q; sparse, row j of item (token, g) is row token h_q + g G + j.  The
    // row part of this lane (its row, or row 0 for rows past M) is fixed, so
    // the loads of a query row take a uniform base and a 32-bit lane offset.
    const int q_lane = [&]() {
      const int r = row_ok ? row : 0;
      if (sparse) return r;
      const int s_tok = r / a.G;
      return s_tok * a.h_q + (r - s_tok * a.G);
    }();
    auto q_item = [&](int item) __attribute__((always_inline)) -> int64_t {
      const int tok_or_b = div_by(item, (unsigned)a.h_kv, a.head_mul), kvg = item - tok_or_b * a.h_kv;
      return (int64_t)tok_or_b * (sparse ? a.h_q : a.s_q * a.h_q) + kvg * a.G;
    };
    auto load_q = [&](int item) __attribute__((always_inline)) {
      // global (not generic) pointers: a generic load would also count against
      // the LDS counter and hold up the waits for LDS reads behind it
      typedef const __attribute__((address_space(1))) char gchar;
      typedef const __attribute__((address_space(1))) bf16x8 gbf16x8;
      gchar* qbase = (gchar*)uniform_ptr(reinterpret_cast<const char*>(a.q + q_item(item) * D));
      gchar* qrow = qbase + (unsigned)(q_lane * D * 2);
#pragma unroll
      for (int ks = 0; ks < C::kQf; ++ks) {
        // FP8: the latent k-steps take the values in the order the K reads
        // deliver them (k-step 2 p + e: rows16, lane group g: values
        // 64 p + 16 g + 8 e .. + 7; wide, lane half hl: 32 p + 16 hl + 8 e ..
        // + 7), so that each lane reads 16 codes at once
        const int d0 = kWide ? (KV8 && ks < 32 ? 32 * (ks >> 1) + 16 * hl + 8 * (ks & 1) : 16 * ks + 8 * hl)
                             : (KV8 && ks < 16 ? 64 * (ks >> 1) + 16 * g + 8 * (ks & 1) : 32 * ks + 8 * g);
        qf[ks] = *reinterpret_cast<gbf16x8*>(qrow + 2 * d0);
      }
    };
    // Rows16, dense: the query rows of an item that starts mid-run come in
    // through LDS.  Wave 0 copies them into rows 0..15 of the stage the next
    // tile is headed for (its own share of that tile goes out later, from
    // `off_late`), so no register load has to complete behind a tile copy and
    // the copy of the next tile is not held back at the item boundary.
    Src off_late;
    constexpr int kQLoads = 2 * C::kCG;   // copies of 16 query rows (8 rows x 128 B each)
    auto issue_q = [&](char* stage, int item) __attribute__((always_inline)) {
      const char* q_bytes = reinterpret_cast<const char*>(a.q);
#pragma unroll
      for (int j = 0; j < kQLoads; ++j) {
        const int r = j / C::kCG, cl = j % C::kCG;
        const int qr = cp_row[r] < a.M ? cp_row[r] : 0;     // rows past M borrow row 0
        const char* src = q_bytes + q_row(a, item, qr) * (int64_t)(2 * D) + cl * 128 +
                          (((lane & 7) ^ cp_swz[r]) << 4);
        copy_to_lds_16(src, lds_addr(stage + j * 1024));
      }
    };
    auto q_from_lds = [&](const char* stage) __attribute__((always_inline)) {
      // row li, in the tile layout; fragment ks holds the values load_q puts
      // there: chunk 4 ks + g (FP8 latent k-steps: 8 (ks / 2) + 2 g + ks % 2)
      const int qb = ((li >> 3) * C::kCG << 10) + ((li & 7) << 7);
#pragma unroll
      for (int ks = 0; ks < C::kQf; ++ks) {
        const int c = (KV8 && ks < 16) ? 8 * (ks >> 1) + 2 * g + (ks & 1) : 4 * ks + g;
        qf[ks] = *reinterpret_cast<const bf16x8*>(stage + qb + ((c >> 3) << 10) + (((c & 7) ^ tswz(li)) << 4));
      }
    };
    auto key_limit = [&](int item) __attribute__((always_inline)) -> int {   // dense: keys of this lane's row are < limit
      const int L = item_len(item);
      if (!row_ok) return 0;
      return (!sparse && a.causal) ? L - a.s_q + row / a.G + 1 : L;
    };
    auto rescale = [&](float m_new) __attribute__((always_inline)) {
      const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_ref - m_new);
      l_lane *= alpha;
#pragma unroll
      for (int d = 0; d < 8; ++d) oacc[d] *= alpha;
      m_ref = m_new;
    };

    // Consume one tile held in `stage` (keys blk*64 .. blk*64 + 63 of the item).
    // Wide: if dma_stage is set, the copy of the next tile into it (offsets in
    // `off`) is issued interleaved with the QK^T MFMAs, one instruction every
    // second k-step, so that issuing it never holds the wave up.
    auto compute = [&](const char* stage, const unsigned char* vslot, int blk, int lim,
                       char* dma_stage, auto&& mid) __attribute__((always_inline)) {
      constexpr int kX = kWide ? 16 : 4;     // scores per lane
      float x[kX];                           // raw scores of the lane's keys, -inf where masked
      float mx;                              // raw row max over this wave's keys
      if constexpr (!kWide) {
        // S^T (16 keys x 16 rows): all kQf K fragments first, one LDS latency for the chain.
        floatx4 sacc = floatx4{0.f, 0.f, 0.f, 0.f};
        bf16x8 kf[C::kQf];
        if constexpr (KV8) {
#pragma unroll
          for (int p = 0; p < 8; ++p) {   // 16 codes: values 64 p + 16 g .. + 15, k-steps 2 p and 2 p + 1
            const i32x4 u = *reinterpret_cast<const i32x4*>(stage + k8_base + ((p >> 1) << 10) + k8_x[p & 1]);
            kf[2 * p] = fp8x8_to_bf16(__builtin_shufflevector(u, u, 0, 1));
            kf[2 * p + 1] = fp8x8_to_bf16(__builtin_shufflevector(u, u, 2, 3));
          }
#pragma unroll
          for (int ks = 16; ks < 18; ++ks)
            kf[ks] = *reinterpret_cast<const bf16x8*>(stage + k8_base + r8_x[ks - 16]);
        } else {
#pragma unroll
          for (int ks = 0; ks < C::kQf; ++ks)
            kf[ks] = *reinterpret_cast<const bf16x8*>(stage + k_base + ((ks >> 1) << 10) + k_x[ks & 1]);
        }
        // element i: key 16 tg + 4 g + i
        const int t0 = 16 * tg + 4 * g;
        if constexpr (!KV8) {
#pragma unroll
          for (int ks = 0; ks < C::kQf; ++ks) sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks], qf[ks], sacc, 0, 0, 0);
        } else {
          // one accumulation per 128-value latent block (4 k-steps each), then
          // the keys' block scales; the RoPE k-steps 16, 17 are not scaled
          floatx4 sb[4];
#pragma unroll
          for (int b = 0; b < 4; ++b) sb[b] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 16; ++ks)
            sb[ks >> 2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks], qf[ks], sb[ks >> 2], 0, 0, 0);
#pragma unroll
          for (int ks = 16; ks < 18; ++ks) sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks], qf[ks], sacc, 0, 0, 0);
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const floatx4 sc = *reinterpret_cast<const floatx4*>(sc_tab + 64 * b + t0);
#pragma unroll
            for (int i = 0; i < 4; ++i) sacc[i] = __builtin_fmaf(sc[i], sb[b][i], sacc[i]);
          }
        }
        unsigned vb = 0;
        if constexpr (sparse) vb = *reinterpret_cast<const unsigned*>(vslot + t0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bool ok;
          if constexpr (sparse) ok = row_ok && ((vb >> (8 * i)) & 0xff);
          else ok = blk * kPage + t0 + i < lim;
          x[i] = ok ? sacc[i] : -INFINITY;
        }
        mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        mx = xor32_max(xor16_max(mx));
      } else {
        // S^T (32 keys x 32 rows) = K Q^T over kQf k-steps of 16.  The loop is
        // written twice so that issuing the next tile's copy inside it costs
        // no branch per k-step.
        floatx16 sacc = {};
        floatx16 sblk[KV8 ? 4 : 1] = {};   // FP8: one accumulation per latent block
        auto qk = [&](auto with_dma) __attribute__((always_inline)) {
          constexpr int kPre = 6;
          // K fragment of k-step ks: bf16 values; FP8: for an even latent
          // k-step the 16 codes of k-steps ks and ks + 1 (values 16 ks + 16 hl
          // .. + 15, one chunk; the query fragments follow the same order),
          // nothing for an odd one, 8 bf16 values for a RoPE k-step
          auto kread = [&](int ks) __attribute__((always_inline)) -> i32x4 {
            if constexpr (KV8) {
              if (ks < 32) {
                if (ks & 1) return i32x4{};
                return *reinterpret_cast<const i32x4*>(stage + k8_base + ((ks >> 3) << 10) +
                                                       (((2 * ((ks >> 1) & 3) + hl) ^ k8_sw) << 4));
              }
              return *reinterpret_cast<const i32x4*>(stage + k8_base + (4 << 10) +
                                                     (((2 * (ks - 32) + hl) ^ k8_sw) << 4));
            } else {
              return *reinterpret_cast<const i32x4*>(stage + k_base + ((ks >> 2) << 10) + k_x[ks & 3]);
            }
          };
          i32x2 khi = {0, 0};   // FP8: the upper 8 codes of the last even latent read
          auto kuse = [&](int ks, i32x4 v) __attribute__((always_inline)) -> bf16x8 {
            if constexpr (KV8) {
              if (ks < 32) {
                if (ks & 1) return fp8x8_to_bf16(khi);
                khi = __builtin_shufflevector(v, v, 2, 3);
                return fp8x8_to_bf16(__builtin_shufflevector(v, v, 0, 1));
              }
            }
            return __builtin_bit_cast(bf16x8, v);
          };
          i32x4 kf[kPre];
#pragma unroll
          for (int ks = 0; ks < kPre; ++ks) kf[ks] = kread(ks);
          static_for<C::kQf>([&](auto ksc) __attribute__((always_inline)) {
            constexpr int ks = decltype(ksc)::value;
            const bf16x8 kcur = kuse(ks, kf[ks % kPre]);
            if constexpr (ks + kPre < C::kQf) kf[ks % kPre] = kread(ks + kPre);
            // FP8: each latent block (k-steps 8 b .. 8 b + 7) accumulates on
            // its own; the RoPE k-steps go into sacc
            if constexpr (KV8) {
              if constexpr (ks < 32) sblk[ks >> 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kcur, qf[ks], sblk[ks >> 3], 0, 0, 0);
              else sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kcur, qf[ks], sacc, 0, 0, 0);
            } else {
              sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kcur, qf[ks], sacc, 0, 0, 0);
            }
            if constexpr (decltype(with_dma)::value) {
              // one copy every second k-step
              static_assert(2 * C::kLoads <= C::kQf, "the copies must fit the k-steps");
              if constexpr (ks % 2 == 0 && ks / 2 < C::kLoads)
                issue_one(dma_stage, off, std::integral_constant<int, ks / 2>{});
            }
            // work for later tiles placed between MFMAs of the chain, where
            // the wave has issue slots to spare
            if constexpr (ks == 8) mid();
            __builtin_amdgcn_sched_barrier(0);   // keep the reads kPre MFMAs ahead
          });
        };
        if (dma_stage != nullptr) qk(std::true_type{});
        else qk(std::false_type{});
        if constexpr (KV8) {
#pragma unroll
          for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const floatx4 sc = *reinterpret_cast<const floatx4*>(sc_tab + 64 * b + 32 * half + 8 * q4 + 4 * hl);
#pragma unroll
              for (int i = 0; i < 4; ++i) sacc[4 * q4 + i] = __builtin_fmaf(sc[i], sblk[b][4 * q4 + i], sacc[4 * q4 + i]);
            }
        }
        // element r: key 32 half + 8 (r / 4) + 4 hl + r % 4.  Tiles whose keys
        // are all valid for every row of the wave skip the per-key mask.
        const bool full = !sparse && __builtin_amdgcn_ballot_w64(blk * kPage + 32 * half + 32 <= lim) ==
                                         __builtin_amdgcn_read_exec();
        if (full) {
#pragma unroll
          for (int r = 0; r < 16; ++r) x[r] = sacc[r];
        } else {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int t0 = 32 * half + 8 * q4 + 4 * hl;
            unsigned vb = 0;
            if constexpr (sparse) vb = *reinterpret_cast<const unsigned*>(vslot + t0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              bool ok;
              if constexpr (sparse) ok = row_ok && ((vb >> (8 * i)) & 0xff);
              else ok = blk * kPage + t0 + i < lim;
              x[4 * q4 + i] = ok ? sacc[4 * q4 + i] : -INFINITY;
            }
          }
        }
        mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
        mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(x[8], x[9]), fmaxf(x[10], x[11])),
                             fmaxf(fmaxf(x[12], x[13]), fmaxf(x[14], x[15]))));
        mx = xor32_max(mx);
      }
      mx *= a.scale_log2;    // scale > 0: the max of the scaled scores

      // Probabilities against the current reference, published with the row
      // maxima; the waves holding a row then see its maxima over the whole
      // tile and move the reference together (when the row outgrew it by 2^8),
      // recomputing and republishing the probabilities.  The decision to take
      // that path is the same in every wave of the workgroup.
      float p[kX];
      bf16x8 pown[kWide ? 2 : 1];   // wide: the lane's bf16 probabilities, PV k-steps 2 half + m
      auto probs = [&]() __attribute__((always_inline)) {
        const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
#pragma unroll
        for (int i = 0; i < kX; ++i) p[i] = fast_exp2(__builtin_fmaf(x[i], a.scale_log2, -m_use));
      };
      auto publish = [&]() __attribute__((always_inline)) {
        if constexpr (!kWide) {
          bf16x4 pv;
#pragma unroll
          for (int i = 0; i < 4; ++i) pv[i] = (__bf16)p[i];
          // FP8 keeps the keys of a (c, g) slot group in natural order (key
          // 32 c + 8 g + j in slot j), as its transposed V^T reads deliver them
          if constexpr (KV8)
            *reinterpret_cast<bf16x4*>(pbuf + li * kPRow + (tg >> 1) * 64 + (2 * (tg & 1) + (g >> 1)) * 16 + (g & 1) * 8) = pv;
          else
            *reinterpret_cast<bf16x4*>(pbuf + li * kPRow + (tg >> 1) * 64 + g * 16 + (tg & 1) * 8) = pv;
        } else if constexpr (KV8) {
          // FP8: natural key order, as the transposed V^T reads deliver the
          // keys: k-step 2 half + m, key 16 (2 half + m) + 8 q + 4 hl + i (score
          // element 8 m + 4 q + i of this lane) goes to slot 4 hl + i of lane
          // 32 q + lrow
#pragma unroll
          for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              bf16x4 v;
#pragma unroll
              for (int i = 0; i < 4; ++i) v[i] = (__bf16)p[8 * m + 4 * q + i];
              *reinterpret_cast<bf16x4*>(pbuf + ((wave * 2 + m) * 64 + 32 * q + lrow) * 16 + 8 * hl) = v;
            }
        } else {
#pragma unroll
          for (int m = 0; m < 2; ++m) {
#pragma unroll
            for (int i = 0; i < 8; ++i) pown[m][i] = (__bf16)p[8 * m + i];
            *reinterpret_cast<bf16x8*>(pbuf + ((wave * 2 + m) * 64 + lane) * 16) = pown[m];
          }
        }
      };
      probs();
      publish();
      if (lane < kRw) red_m[wave][lane] = mx;
      if constexpr (kWide) {
        const bool need = __builtin_amdgcn_ballot_w64(mx > m_ref + kLazy) != 0;   // all lanes vote
        if (lane == 0) red_need[wave] = need;
      }
      barrier_keep_loads();
      if constexpr (!kWide) {
        // every wave has read the query rows staged in `dma_stage`
        if (dma_stage != nullptr) issue(dma_stage, off_late);
      }
      float m_tile;
      bool move;
      if constexpr (!kWide) {
        m_tile = red_m[0][li];
#pragma unroll
        for (int j = 1; j < 4; ++j) m_tile = fmaxf(m_tile, red_m[j][li]);
        move = __builtin_amdgcn_ballot_w64(m_tile > m_ref + kLazy) != 0;   // same in every wave
      } else {
        m_tile = fmaxf(red_m[2 * pair][lrow], red_m[2 * pair + 1][lrow]);
        move = (red_need[0] | red_need[1] | red_need[2] | red_need[3]) != 0;
      }
      if (move) {
        rescale(fmaxf(m_ref, m_tile));
        probs();
        publish();
        barrier_keep_loads();
      }
#pragma unroll
      for (int i = 0; i < kX; ++i) l_lane += p[i];

      if constexpr (!kWide) {
        // O^T += V^T P^T over the 64 keys, 32 at a time: slots 0..3 of lane
        // group g are keys 4 g + i of subtile 2 c, slots 4..7 those of 2 c + 1.
        // 16 MFMAs, (c, dt) in order; the V^T fragments are read kPv MFMAs ahead.
        bf16x8 pb[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) pb[c] = *reinterpret_cast<const bf16x8*>(pbuf + li * kPRow + c * 64 + g * 16);
        if constexpr (KV8) {
          // the wave's output columns are latent block tg: each key's scale for it
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const floatx4 s0 = *reinterpret_cast<const floatx4*>(sc_tab + 64 * tg + 32 * c + 8 * g);
            const floatx4 s1 = *reinterpret_cast<const floatx4*>(sc_tab + 64 * tg + 32 * c + 8 * g + 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              pb[c][i] = (__bf16)((float)pb[c][i] * s0[i]);
              pb[c][4 + i] = (__bf16)((float)pb[c][4 + i] * s1[i]);
            }
          }
        }
        constexpr int kPv = 6;
        if constexpr (KV8) {
          // V^T fragments (16 columns x 32 keys) by transposed 8-bit reads of
          // the copied codes, converted in registers; keys in natural order
          auto v8addr = [&](int n) __attribute__((always_inline)) -> const char* {
            const int c = n >> 3, dt = n & 7;
            return stage + v8_base + c * (20 << 10) + ((dt ^ v8_sw) << 4);
          };
          i32x2 vr[kPv];
#pragma unroll
          for (int n = 0; n < kPv; ++n) vr[n] = read_tr8(v8addr(n));
#pragma unroll
          for (int n = 0; n < 16; ++n) {
            const bf16x8 va = fp8x8_to_bf16(vr[n % kPv]);
            if (n + kPv < 16) vr[n % kPv] = read_tr8(v8addr(n + kPv));
            oacc[n & 7] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[n >> 3], oacc[n & 7], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);   // keep the reads kPv MFMAs ahead
          }
        } else {
        auto vaddr = [&](int n, int e) __attribute__((always_inline)) -> const char* {
          const int c = n >> 3, dt = n & 7;
          return stage + v_base + (2 * c + e) * (2 * C::kCG * 1024) + ((dt >> 2) << 10) + v_x[0][dt & 3];
        };
        bf16x4 vq0[kPv], vq1[kPv];
#pragma unroll
        for (int n = 0; n < kPv; ++n) {
          vq0[n] = read_tr(vaddr(n, 0));
          vq1[n] = read_tr(vaddr(n, 1));
        }
#pragma unroll
        for (int n = 0; n < 16; ++n) {
          const bf16x8 va = __builtin_shufflevector(vq0[n % kPv], vq1[n % kPv], 0, 1, 2, 3, 4, 5, 6, 7);
          if (n + kPv < 16) {
            vq0[n % kPv] = read_tr(vaddr(n + kPv, 0));
            vq1[n % kPv] = read_tr(vaddr(n + kPv, 1));
          }
          oacc[n & 7] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[n >> 3], oacc[n & 7], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);   // keep the reads kPv MFMAs ahead
        }
        }
      } else {
        // O^T += V^T P^T over the 64 keys in k-steps of 16.  k-step j = 2 kb + m
        // holds, for lane half hl, keys 16 j + 4 hl + i (slots 0..3) and
        // 16 j + 8 + 4 hl + i (slots 4..7): exactly score elements 8 m .. 8 m + 7
        // of the same lane in the wave with half == kb.
        bf16x8 pb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int owner = (j >> 1) == half ? wave : (wave ^ 1);
          if constexpr (KV8)   // FP8: both halves through LDS, in natural key order
            pb[j] = *reinterpret_cast<const bf16x8*>(pbuf + ((owner * 2 + (j & 1)) * 64 + lane) * 16);
          else
            pb[j] = (j >> 1) == half ? pown[j & 1]
                                     : *reinterpret_cast<const bf16x8*>(pbuf + ((owner * 2 + (j & 1)) * 64 + lane) * 16);
        }
        // 32 MFMAs, (j, db) in order; the V^T fragments are read kPv MFMAs ahead.
        constexpr int kPv = 6;
        if constexpr (KV8) {
          // V^T fragments by transposed 8-bit reads of the codes, converted in
          // registers; P scaled by the keys' scales of the columns' latent
          // block 2 half + db / 4
          auto v8addr = [&](int n) __attribute__((always_inline)) -> const char* {
            const int j = n >> 3, db = n & 7;
            return stage + v8_base + ((10 * j + (db >> 2)) << 10) + v8_x[db & 3];
          };
          i32x2 vr[kPv];
#pragma unroll
          for (int n = 0; n < kPv; ++n) vr[n] = read_tr8(v8addr(n));
          bf16x8 pbs;   // scaled probabilities of the current (k-step, block)
#pragma unroll
          for (int n = 0; n < 32; ++n) {
            const bf16x8 va = fp8x8_to_bf16(vr[n % kPv]);
            if (n + kPv < 32) vr[n % kPv] = read_tr8(v8addr(n + kPv));
            if ((n & 3) == 0) {
              const bf16x8 pbn = pb[n >> 3];
              const float* st = sc_tab + 64 * (2 * half + ((n & 7) >> 2)) + 16 * (n >> 3) + 8 * hl;
              const floatx4 s0 = *reinterpret_cast<const floatx4*>(st);
              const floatx4 s1 = *reinterpret_cast<const floatx4*>(st + 4);
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                pbs[i] = (__bf16)((float)pbn[i] * s0[i]);
                pbs[4 + i] = (__bf16)((float)pbn[4 + i] * s1[i]);
              }
            }
            oacc[n & 7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pbs, oacc[n & 7], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);   // keep the reads kPv MFMAs ahead
          }
        } else {
          auto vaddr = [&](int n, int e) __attribute__((always_inline)) -> const char* {
            const int j = n >> 3, db = n & 7;
            return stage + v_base + (2 * j + e) * (C::kCG * 1024) + ((db >> 1) << 10) + v_x[e][db & 1];
          };
          bf16x4 vq0[kPv], vq1[kPv];
#pragma unroll
          for (int n = 0; n < kPv; ++n) {
            vq0[n] = read_tr(vaddr(n, 0));
            vq1[n] = read_tr(vaddr(n, 1));
          }
#pragma unroll
          for (int n = 0; n < 32; ++n) {
            const bf16x8 va = __builtin_shufflevector(vq0[n % kPv], vq1[n % kPv], 0, 1, 2, 3, 4, 5, 6, 7);
            if (n + kPv < 32) {
              vq0[n % kPv] = read_tr(vaddr(n + kPv, 0));
              vq1[n % kPv] = read_tr(vaddr(n + kPv, 1));
            }
            oacc[n & 7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[n >> 3], oacc[n & 7], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);   // keep the reads kPv MFMAs ahead
          }
        }
      }
    };

    // 128-row variant: the wave's 32 query rows against all 64 keys of the
    // tile.  S^T block kb (keys 32 kb .. 32 kb + 31) x 32 rows over kQf k-steps
    // of 16 (v_mfma_f32_32x32x16_bf16), block 0 then block 1; then
    // the softmax of the wave's own rows, which needs no other wave (each lane
    // holds 16 keys of each block for its row, its partner lane ^ 32 the other
    // 16); then O^T += V^T P^T over 4 k-steps of 16 keys and the 16 column
    // blocks of 32.  hook(n) runs after QK^T MFMA n (the caller does the index
    // work for later tiles at the first ones); the copy of the next tile
    // (dma_stage, `off`) follows, one instruction every third QK^T MFMA;
    // after_qk() runs once the query fragments are no longer needed for this
    // tile.  all_valid: every key of a sparse tile is valid (no mask).
    auto compute_full = [&](const char* stage, const unsigned char* vslot, bool all_valid, int blk, int lim,
                            char* dma_stage, auto&& hook, auto&& after_qk, bool first) __attribute__((always_inline)) {
      if constexpr (kFull) {
        floatx16 sacc[2];
        // QK^T MFMAs: k-step n % kQf of block n / kQf.  One block after the
        // other: the first block's scores leave the accumulation registers
        // while the second accumulates, so that only one block's worth of
        // them is needed beside the output accumulators.
        constexpr int kN = 2 * C::kQf;
        constexpr int kPre = 4;             // K fragments read ahead
        // The copies of the next tile go out one every third MFMA from MFMA
        // kCopy0 on; the index work for later tiles (hook(n), at the first
        // MFMAs) comes first, so that a wait it may contain never waits for
        // this tile's copies.
        constexpr int kCopy0 = 16;
        static_assert(kCopy0 + 3 * (C::kLoads - 1) < kN, "the copies must fit the QK^T MFMAs");
        auto kread = [&](int n) __attribute__((always_inline)) -> bf16x8 {
          const int ks = n % C::kQf, kb = n / C::kQf;
          return *reinterpret_cast<const bf16x8*>(stage + k_base + kb * ((4 * C::kCG) << 10) +
                                                  ((ks >> 2) << 10) + k_x[ks & 3]);
        };
        auto qk = [&](auto with_dma) __attribute__((always_inline)) {
          bf16x8 kf[kPre];
          static_for<kPre>([&](auto nc) __attribute__((always_inline)) { kf[decltype(nc)::value] = kread(decltype(nc)::value); });
          static_for<kN>([&](auto nc) __attribute__((always_inline)) {
            constexpr int n = decltype(nc)::value;
            const bf16x8 kc = kf[n % kPre];
            if constexpr (n + kPre < kN) kf[n % kPre] = kread(n + kPre);
            if constexpr (n % C::kQf == 0) sacc[n / C::kQf] = mfma_v0(kc, qf[0]);
            else mfma_v(sacc[n / C::kQf], kc, qf[n % C::kQf]);
            hook(nc);
            if constexpr (decltype(with_dma)::value && n >= kCopy0 && (n - kCopy0) % 3 == 0 &&
                          (n - kCopy0) / 3 < C::kLoads)
              issue_one(dma_stage, off, std::integral_constant<int, (n - kCopy0) / 3>{});
            __builtin_amdgcn_sched_barrier(0);   // keep the reads kPre MFMAs ahead
          });
        };
        if (dma_stage != nullptr) qk(std::true_type{});
        else qk(std::false_type{});
        mfma_result_wait();
        after_qk();
        // element r of block kb: key 32 kb + 8 (r / 4) + 4 hl + r % 4.  Tiles
        // whose keys are all valid for every row of the wave skip the mask.
        const bool full = sparse ? all_valid && __builtin_amdgcn_ballot_w64(row_ok) == __builtin_amdgcn_read_exec()
                                 : __builtin_amdgcn_ballot_w64(blk * kPage + kPage <= lim) ==
                                       __builtin_amdgcn_read_exec();
        if (!full) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const int t0 = 32 * kb + 8 * q4 + 4 * hl;
              unsigned vb = 0;
              if constexpr (sparse) vb = *reinterpret_cast<const unsigned*>(vslot + t0);
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                bool ok;
                if constexpr (sparse) ok = row_ok && ((vb >> (8 * i)) & 0xff);
                else ok = blk * kPage + t0 + i < lim;
                if (!ok) sacc[kb][4 * q4 + i] = -INFINITY;
              }
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; r += 4)
            mx = fmaxf(mx, fmaxf(fmaxf(sacc[kb][r], sacc[kb][r + 1]), fmaxf(sacc[kb][r + 2], sacc[kb][r + 3])));
        mx = xor32_max(mx) * a.scale_log2;   // scale > 0: the max of the scaled scores
        // The first tile of a run sets the reference (O and l start at zero:
        // the run's first PV MFMAs take a zero accumulator).  Later, the
        // reference of the wave's rows moves when one of them outgrew it by
        // 2^8 (all rows of the wave move together, each to its own max).
        if (first) {
          m_ref = mx;
        } else if (__builtin_amdgcn_ballot_w64(mx > m_ref + kLazy) != 0) {
          const float m_new = fmaxf(m_ref, mx);
          const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_ref - m_new);
#pragma unroll
          for (int d = 0; d < 16; ++d) scale_agpr_block(oacc[d], alpha);
          l_lane *= alpha;
          m_ref = m_new;
        }
        const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
        // P^T for PV k-step j = 2 kb + m: elements 8 m .. 8 m + 7 of block kb,
        // i.e. keys 16 j + 4 hl + i (slots 0..3) and 16 j + 8 + 4 hl + i
        // (slots 4..7), the order the V^T reads deliver
        bf16x8 pb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float pv = fast_exp2(__builtin_fmaf(sacc[j >> 1][8 * (j & 1) + i], a.scale_log2, -m_use));
            l_lane += pv;
            pb[j][i] = (__bf16)pv;
          }
        // O^T += V^T P^T: MFMA n = 16 j + db (k-step j, column block db); the
        // V^T fragments are read kPv MFMAs ahead.
        constexpr int kPv = 4;
        auto vaddr = [&](int n, int e) __attribute__((always_inline)) -> const char* {
          const int j = n >> 4, db = n & 15;
          return stage + v_base + (2 * j + e) * (C::kCG * 1024) + ((db >> 1) << 10) + v_x[e][db & 1];
        };
        bf16x4 vq0[kPv], vq1[kPv];
        static_for<kPv>([&](auto nc) __attribute__((always_inline)) {
          constexpr int n = decltype(nc)::value;
          vq0[n] = read_tr(vaddr(n, 0));
          vq1[n] = read_tr(vaddr(n, 1));
        });
        auto pv = [&](auto first_c) __attribute__((always_inline)) {
          static_for<64>([&](auto nc) __attribute__((always_inline)) {
            constexpr int n = decltype(nc)::value;
            const bf16x8 va = __builtin_shufflevector(vq0[n % kPv], vq1[n % kPv], 0, 1, 2, 3, 4, 5, 6, 7);
            if constexpr (n + kPv < 64) {
              vq0[n % kPv] = read_tr(vaddr(n + kPv, 0));
              vq1[n % kPv] = read_tr(vaddr(n + kPv, 1));
            }
            if constexpr (decltype(first_c)::value && n < 16)
              oacc[n & 15] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[0], floatx16{}, 0, 0, 0);
            else
              oacc[n & 15] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[n >> 4], oacc[n & 15], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);   // keep the reads kPv MFMAs ahead
          });
        };
        pv(std::false_type{});
      }
    };

    // Finish the run of `item`: write O/LSE, or the partial (bf16 O, fp32
    // LSE) when the item is split over several runs.
    int merge_item[2] = {-1, -1};   // single launch: split items whose partials this workgroup merges
    int n_merge = 0;
    auto finish = [&](int item, int split) __attribute__((always_inline)) {
      int slot0, slot1;
      if (item - it_first < 63) {
        slot0 = __builtin_amdgcn_readlane(splits_v, item - it_first);
        slot1 = __builtin_amdgcn_readlane(splits_v, item - it_first + 1);
      } else {
        read_scalar2(a.num_splits + item, a.num_splits + item + 1, slot0, slot1);
      }
      const int nsplit = slot1 - slot0;
      const bool final_out = nsplit == 1;
      const int64_t part_base = (int64_t)(slot0 + split) * a.part_rows;
      // row sums over the lanes and waves holding the row (same order everywhere)
      float l_tot = l_lane;
      if constexpr (!kWide) l_tot = xor16_sum(l_tot);
      l_tot = xor32_sum(l_tot);
      if constexpr (!kFull) {   // the 128-row variant holds each row in one wave
        if (lane < kRw) red_l[wave][lane] = l_tot;
        barrier_keep_loads();
        if constexpr (!kWide) {
          l_tot = red_l[0][li];
#pragma unroll
          for (int j = 1; j < 4; ++j) l_tot += red_l[j][li];
        } else {
          l_tot = red_l[2 * pair][lrow] + red_l[2 * pair + 1][lrow];
        }
      }
      if (row_ok) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        const int64_t orow = final_out ? q_row(a, item, row) : part_base + row;
        // element (d, i) of the lane: column c0 + 16 d + 4 g + i (rows16),
        // c0 + 32 d + 8 (i / 4) + 4 hl + i % 4 (wide; 16 blocks d in the
        // 128-row variant)
        const int c0 = kWide ? 256 * half + 4 * hl : 128 * tg + 4 * g;
        if (final_out) {
          uint16_t* orp = a.o + orow * kDv + c0;
#pragma unroll
          for (int d = 0; d < kOBlocks; ++d)
#pragma unroll
            for (int q4 = 0; q4 < (kWide ? 4 : 1); ++q4) {
              bf16x4 v;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                float e = oacc[d][4 * q4 + i];
                if constexpr (kFull) e = agpr_read(e);
                v[i] = (__bf16)(e * inv);
              }
              *reinterpret_cast<bf16x4*>(orp + (kWide ? 32 * d + 8 * q4 : 16 * d)) = v;
              if constexpr (kFull) __builtin_amdgcn_sched_barrier(0);   // one block's registers at a time
            }
        } else {
          uint16_t* orp = a.part_o + orow * kDv + c0;
          // 128-row variant, two launches: the wave's 32 rows as one block of
          // 16384 values in accumulator order (value i of piece (d, q4) of
          // lane l at ((4 d + q4) * 64 + l) * 4 + i), so that every store
          // instruction writes 512 contiguous bytes; combine_kernel reads the
          // blocks back.
          uint16_t* blk = a.part_o + (part_base + row0 + 32 * pair) * kDv + 4 * lane;
#pragma unroll
          for (int d = 0; d < kOBlocks; ++d)
#pragma unroll
            for (int q4 = 0; q4 < (kWide ? 4 : 1); ++q4) {
              bf16x4 v;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                float e = oacc[d][4 * q4 + i];
                if constexpr (kFull) e = agpr_read(e);
                v[i] = (__bf16)(e * inv);
              }
              uint16_t* dst = (kFull && !FUSED) ? blk + (4 * d + q4) * 256 : orp + (kWide ? 32 * d + 8 * q4 : 16 * d);
              if constexpr (FUSED) store_part4_agent(dst, v);
              else *reinterpret_cast<bf16x4*>(dst) = v;
              if constexpr (kFull) __builtin_amdgcn_sched_barrier(0);
            }
        }
        const bool lse_lane = kWide ? (half == 0 && hl == 0) : (tg == 0 && g == 0);
        if (lse_lane) {
          const float lse = l_tot > 0.f ? m_ref * kLn2 + logf(l_tot) : -INFINITY;
          if (final_out) a.lse[orow] = lse;
          else if (FUSED) store_part1_agent(a.part_lse + orow, lse);
          else a.part_lse[orow] = lse;
        }
      }
      if (FUSED && !final_out) {
        // Single launch: count this run in.  The last run of the item (and
        // row tile) to arrive merges the partials once its own tile stream is
        // done (a worker has at most two split runs: its first and its last
        // item).  Every wave's partial stores are complete before the count
        // is raised.
        __builtin_amdgcn_s_waitcnt(0);
        barrier_keep_loads();
        if (threadIdx.x == 0)
          red_need[0] = __hip_atomic_fetch_add(a.arrivals + (int64_t)item * a.m_tiles + mt, 1,
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        barrier_keep_loads();
        if (red_need[0] == nsplit - 1) {
          merge_item[n_merge] = item;
          ++n_merge;
        }
        barrier_keep_loads();   // red_need is reused by the next tile's softmax
      }
      // reset for the next run (the 128-row variant's first PV MFMAs of a run
      // take a zero accumulator instead)
      if constexpr (!kFull) {
#pragma unroll
        for (int d = 0; d < kOBlocks; ++d) oacc[d] = Acc{};
      }
      m_ref = -INFINITY;
      l_lane = 0.f;
    };

    // ---- the tile stream ----
    int cur_item = it_first, cur_blk = blk_first;
    int t = 0;   // tile counter (validity slot t & 3)
    if constexpr (!kFull) {
#pragma unroll
      for (int d = 0; d < kOBlocks; ++d) oacc[d] = Acc{};
    }
    // Prologue.  The loads the compiler tracks (lengths, index data of tile 0,
    // the first query rows) go out together and are waited for before the
    // first copy is issued: a tracked load still pending behind a copy would
    // make its first use wait for the copy as well.
    TileRaw raw;
    if constexpr (sparse) tile_fetch(cur_item, cur_blk, raw);
    load_q(cur_item);
    {
      const int seq = item_seq(a, cur_item);
      read_scalar2(a.seqlens + seq, a.block_table + (int64_t)seq * a.max_blocks + (sparse ? 0 : cur_blk),
                   len_first, page_first);
    }
    if constexpr (!sparse) raw.v[0] = page_first;
    int cur_hi = seg_hi(cur_item);
    int nx_item, nx_blk, nx_hi;
    advance(cur_item, cur_blk, cur_hi, nx_item, nx_blk, nx_hi);
    int cur_lim = key_limit(cur_item);
    int cur_split = split_first;
    // Wide, sparse: tile 1's index entries come in with tile 0's, and tile 1
    // is translated here (its pages are copied in before the first copy)
    if constexpr (kWide && sparse) {
      if (nx_item >= 0) idx_dma(nx_item, nx_blk, 1);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    if constexpr (kWide && sparse) {
      barrier_keep_loads();                 // tile 1's entries, copied by wave 0, for every wave
      if (nx_item >= 0) translate_lds(nx_item, nx_blk, 1, kvalid[1]);
    }
    tile_finish(cur_item, cur_blk, raw, off, kvalid[0]);
    issue(s0, off);
    if constexpr (kWide && sparse) {
      int p_item = -1, p_blk = 0, p_hi = 0;   // tile 2: its index entries into the ring
      if (nx_item >= 0) advance(nx_item, nx_blk, nx_hi, p_item, p_blk, p_hi);
      if (p_item >= 0) idx_dma(p_item, p_blk, 2);
    } else if constexpr (kWide) {
      if (nx_item >= 0) idx_dma(nx_item, nx_blk, 1);   // tile 1's offsets are made in step 0
    } else if (nx_item >= 0) {
      tile_fetch(nx_item, nx_blk, raw);
      if constexpr (sparse) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      tile_finish(nx_item, nx_blk, raw, off, kvalid[1]);
    }

    bool q_pending = false;   // rows16, dense: the query rows of tile t's item come through LDS
    bool q8_pending = false;  // rows16, FP8: they wait in qbuf[q8_rd]
    int q8_wr = 0, q8_rd = 0;

    // One step: tile t sits in `cur`; tile t + 1 goes into `nxt`.  Tile t + 1
    // is requested before waiting for tile t, so two tiles are in flight while
    // a wave waits; the wait below counts only this wave's copy of tile t + 1
    // as still outstanding (memory loads complete in order).
    auto step = [&](char* cur, char* nxt) __attribute__((always_inline)) -> bool {
      const bool has_next = nx_item >= 0;
      int n2_item = -1, n2_blk = 0, n2_hi = 0;
      if (has_next) advance(nx_item, nx_blk, nx_hi, n2_item, n2_blk, n2_hi);
      if constexpr (kWide) {
        // Tile t was requested during the previous step's QK^T (and before it
        // the index data of a later tile; sparse: the block-table entries of
        // tile t + 1): nothing else is in flight.
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        barrier_keep_loads();          // tile t in LDS for every wave; every wave is done with `nxt`
        if constexpr (KV8) sc_tab = reinterpret_cast<const float*>(cur + kRaw8ScaleOff);   // operands read from the codes
        // Tile t + 1's offsets (its copy goes out during QK^T).  Sparse: from
        // its entries and pages, copied in during the last step.
        if constexpr (sparse) {
          if (has_next) finish_lds(nx_item, nx_blk, t + 1, off);
        } else if (has_next) {
          idx_from_lds(nx_item, nx_blk, t + 1, raw);
          tile_finish(nx_item, nx_blk, raw, off, kvalid[(t + 1) & 3]);
        }
        // Work for later tiles, done between QK^T MFMAs: sparse, tile t + 2's
        // pages and validity and tile t + 3's index entries; dense, tile
        // t + 2's page id.
        auto mid = [&]() __attribute__((always_inline)) {
          if (n2_item < 0) return;
          if constexpr (sparse) {
            translate_lds(n2_item, n2_blk, t + 2, kvalid[(t + 2) & 3]);
            int n3_item = -1, n3_blk = 0, n3_hi = 0;
            advance(n2_item, n2_blk, n2_hi, n3_item, n3_blk, n3_hi);
            if (n3_item >= 0) idx_dma(n3_item, n3_blk, t + 3);
          } else {
            idx_dma(n2_item, n2_blk, t + 2);
          }
        };
        const bool ends = !has_next || nx_item != cur_item;
        if constexpr (sparse) {
          bool any_v, all_v;
          tile_validity(kvalid[t & 3], any_v, all_v);
          clear_if_empty(cur, any_v);
        }
        if constexpr (!kFull) compute(cur, kvalid[t & 3], cur_blk, cur_lim, has_next ? nxt : nullptr, mid);
        if (ends) {
          finish(cur_item, cur_split);
          if (has_next) {
            cur_lim = key_limit(nx_item);
            cur_split = 0;
            load_q(nx_item);     // completed here (see the prologue)
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
          }
        }
        cur_item = nx_item;
        cur_blk = nx_blk;
        cur_hi = nx_hi;
        nx_item = n2_item;
        nx_blk = n2_blk;
        nx_hi = n2_hi;
        ++t;
        return has_next;
      }
      barrier_keep_loads();                              // every wave is done with `nxt`
      const bool q_lds = q_pending && wave == 0;         // wave-uniform
      if (q_pending && wave == 0) issue_q(nxt, cur_item);
      if (has_next) {
        if (q_lds) {
          off_late = off;
        } else {
          issue(nxt, off);
        }
      }
      // FP8: tile t + 1 starts an item; its query rows follow the tile's copy
      const bool q8 = kQSlots && has_next && nx_item != cur_item;   // same in every wave
      const int q8_slot = q8_wr;
      if (q8 && wave == 0) issue_q(qbuf[q8_slot], nx_item);
      if (n2_item >= 0) tile_fetch(n2_item, n2_blk, raw);  // index data of tile t + 2
      // Vector-memory operations issued after tile t's copy: the copy of tile
      // t + 1, wave 0's query-row copies (FP8, at an item start) and, in sparse
      // mode, the index loads of tile t + 2.  Waiting until no more than those
      // are outstanding completes tile t's copy (loads complete in order).  The
      // compiler barrier keeps the index loads above the wait.
      asm volatile("" ::: "memory");
      if (has_next && !q_lds) {
        if (q8 && wave == 0) {
          if (sparse && n2_item >= 0) __builtin_amdgcn_s_waitcnt(waitcnt_vm(C::kLoads + kQLoads + kRaw));
          else __builtin_amdgcn_s_waitcnt(waitcnt_vm(C::kLoads + kQLoads));
        } else if (sparse && n2_item >= 0) {
          __builtin_amdgcn_s_waitcnt(kWaitKeepRawCopy);
        } else {
          __builtin_amdgcn_s_waitcnt(kWaitKeepCopy);
        }
      } else {
        __builtin_amdgcn_s_waitcnt(0);     // wave 0 with staged query rows: tile t, then the rows
      }
      barrier_keep_loads();                              // tile t is in LDS for every wave
      if constexpr (KV8) sc_tab = reinterpret_cast<const float*>(cur + kRaw8ScaleOff);   // operands read from the codes
      if (q_pending) q_from_lds(nxt);
      if (q8_pending) q_from_lds(qbuf[q8_rd]);
      q8_pending = false;
      if (n2_item >= 0) tile_finish(n2_item, n2_blk, raw, off, kvalid[(t + 2) & 3]);
      const bool ends = !has_next || nx_item != cur_item;
      if constexpr (sparse) {
        bool any_v, all_v;
        tile_validity(kvalid[t & 3], any_v, all_v);
        clear_if_empty(cur, any_v);
      }
      compute(cur, kvalid[t & 3], cur_blk, cur_lim, q_lds && has_next ? nxt : nullptr, [] {});
      q_pending = false;
      if (ends) {
        finish(cur_item, cur_split);
        if (has_next) {
          cur_lim = key_limit(nx_item);
          cur_split = 0;
          if constexpr (kQSlots) {
            q8_rd = q8_slot;           // copied in with the next tile
            q8_pending = true;
          } else if constexpr (sparse) {
            // Query rows of the next item, completed before the next copy is
            // issued (see the prologue).
            load_q(nx_item);
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
          } else {
            q_pending = true;          // staged through LDS in the next step
          }
        }
      }
      if (q8) q8_wr ^= 1;
      cur_item = nx_item;
      cur_blk = nx_blk;
      cur_hi = nx_hi;
      nx_item = n2_item;
      nx_blk = n2_blk;
      nx_hi = n2_hi;
      ++t;
      return has_next;
    };
    // 128-row variant: the runs are an outer loop and the tiles of a run an
    // inner one, so that the output accumulators are only read (written out)
    // after the tile loop and stay in their registers across the tiles; the
    // stages alternate by tile number.  The stream of tiles and copies is the
    // same as in the other wide steps: tile t + 1's copy goes out during tile
    // t's QK^T, across run boundaries.
    auto run_full = [&]() __attribute__((always_inline)) {
      bool c_any = true, c_all = true;   // sparse: validity of tile t (any key, every key)
      for (;;) {
        const int run_item = cur_item, run_split = cur_split;
        bool first = true, has_next;
#pragma unroll
        for (int d = 0; d < kOBlocks; ++d)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[d][i] = agpr_zero();
        for (;;) {
          has_next = nx_item >= 0;
          int n2_item = -1, n2_blk = 0, n2_hi = 0;
          if (has_next) advance(nx_item, nx_blk, nx_hi, n2_item, n2_blk, n2_hi);
          // tile t was requested during the previous tile's QK^T: nothing
          // else is in flight
          __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
          barrier_keep_loads();        // tile t in LDS for every wave; every wave is done with `nxt`
          char* cur = (t & 1) ? s1 : s0;
          char* nxt = (t & 1) ? s0 : s1;
          if constexpr (sparse) {
            if (t == 0) tile_validity(kvalid[0], c_any, c_all);
          }
          // Index work for later tiles, between the first QK^T MFMAs, each
          // LDS read a few MFMAs before its result is used: the offsets of
          // tile t + 1 (whose copies start at MFMA 16); sparse, tile t + 2's
          // pages and validity, tile t + 3's index entries and tile t + 1's
          // validity; dense, tile t + 2's page id.
          RowsRaw nr;
          int m_idx = -1;
          bool n_any = true, n_all = true;
          auto hook = [&](auto nc) __attribute__((always_inline)) {
            constexpr int n = decltype(nc)::value;
            if constexpr (n == 0) {
              if (has_next) {
                if constexpr (sparse) finish_read(nx_item, nx_blk, t + 1, nr);
                else nr.idx[0] = idxbuf[(t + 1) & 3][0];
              }
            } else if constexpr (n == 3) {
              if (has_next) {
                if constexpr (sparse) {
                  finish_use(nx_item, nx_blk, nr, off);
                } else {
                  raw.v[0] = nr.idx[0];
                  tile_finish(nx_item, nx_blk, raw, off, kvalid[(t + 1) & 3]);
                }
              }
            } else if constexpr (n == 5) {
              if constexpr (sparse) {
                if (n2_item >= 0) m_idx = translate_read(n2_item, n2_blk, t + 2);
              }
            } else if constexpr (n == 8) {
              if (n2_item >= 0) {
                if constexpr (sparse) {
                  translate_use(n2_item, n2_blk, t + 2, m_idx, kvalid[(t + 2) & 3]);
                  int n3_item = -1, n3_blk = 0, n3_hi = 0;
                  advance(n2_item, n2_blk, n2_hi, n3_item, n3_blk, n3_hi);
                  if (n3_item >= 0) idx_dma(n3_item, n3_blk, t + 3);
                } else {
                  idx_dma(n2_item, n2_blk, t + 2);
                }
              }
            } else if constexpr (n == 10) {
              if constexpr (sparse) {
                if (has_next) tile_validity(kvalid[(t + 1) & 3], n_any, n_all);
              }
            }
          };
          const bool ends = !has_next || nx_item != cur_item;
          clear_if_empty(cur, c_any);
          // The next item's query rows are loaded as soon as this tile's
          // QK^T is done with their registers; they arrive during PV and the
          // end of the run, and the next tile's wait covers them.
          const bool q_next = ends && has_next;
          const int q_item = nx_item;
          compute_full(cur, kvalid[t & 3], c_all, cur_blk, cur_lim, has_next ? nxt : nullptr, hook,
                       [&]() __attribute__((always_inline)) { if (q_next) load_q(q_item); }, first);
          first = false;
          c_any = n_any;
          c_all = n_all;
          cur_item = nx_item;
          cur_blk = nx_blk;
          cur_hi = nx_hi;
          nx_item = n2_item;
          nx_blk = n2_blk;
          nx_hi = n2_hi;
          ++t;
          if (ends) break;
        }
        // The output blocks stay in their AGPRs into the run's end: without
        // this the register allocator moves some of them to VGPRs after the
        // last PV MFMAs, then needs an AGPR back for each read below, parks a
        // whole block in scratch and reloads it behind the partial stores.
#pragma unroll
        for (int d = 0; d < kOBlocks; ++d) asm volatile("" : "+a"(oacc[d]));
        finish(run_item, run_split);
        if (!has_next) break;
        cur_lim = key_limit(cur_item);
        cur_split = 0;
      }
    };
    if constexpr (kFull) {
      run_full();
    } else {
      while (step(s0, s1) && step(s1, s0)) {
      }
    }
    if constexpr (FUSED) {
      // merge the split items whose last run this was, and clear their counts
      for (int k = 0; k < n_merge; ++k) {
        const int item = merge_item[k];
        const int slot0 = a.num_splits[item];
        const int nsplit = a.num_splits[item + 1] - slot0;
        for (int r = wave; r < C::kRows; r += C::kWaves)
          if (row0 + r < a.M) merge_row<true>(a, item, slot0, nsplit, row0 + r, lane);
        if (threadIdx.x == 0)
          __hip_atomic_store(a.arrivals + (int64_t)item * a.m_tiles + mt, 0, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if constexpr (FUSED) {
    // Single launch: items without a key get o = 0, lse = -inf (all their
    // rows), item i from participating workgroup i mod (workers x row tiles).
    const int wid = w * a.m_tiles + mt, nwg = a.num_workers * a.m_tiles;
    for (int i = wid; i < a.num_items; i += nwg) {
      if (a.num_splits[i + 1] == a.num_splits[i])
        for (int r = wave; r < a.M; r += C::kWaves) write_empty_row(a, i, r, lane);
    }
  }
}

template <int V, bool KV8, int D>
hipError_t launch_variant(const DecodeArgs& a, hipStream_t stream) {
  const int groups = (a.num_workers + 7) / 8;
  const int grid = a.m_tiles == 1 ? a.num_workers : groups * 8 * a.m_tiles;
  if (a.fused) {
    if (a.topk > 0)
      hipLaunchKernelGGL((decode_kernel<V, true, KV8, D, true>), dim3(grid), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_kernel<V, false, KV8, D, true>), dim3(grid), dim3(256), 0, stream, a);
  } else if (a.topk > 0) {
    hipLaunchKernelGGL((decode_kernel<V, true, KV8, D, false>), dim3(grid), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL((decode_kernel<V, false, KV8, D, false>), dim3(grid), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace
}  // namespace mla
