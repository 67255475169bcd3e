// StreamKL kernels for gfx950 (AMD Instinct MI355X) and the C ABI declared in streamkl.h.
//
// What is computed (gist.science/pt/paper/2606.20005, "Metodologia" sections 1-3):
//   per (batch, head) slice and query row i, with S_t = scale * Q_t K_t^T,
//   forward:  five running per-row scalars m1, l1, m2, l2, acc over streamed key tiles, then
//             LSE_t = m_t + log l_t,  KL = acc / l1 + LSE2 - LSE1;
//   backward: P_t = exp(S_t - LSE_t) regenerated tile by tile from the saved LSEs, then
//             setting 1 (P1 fixed): dS2 = g (P2 - P1);
//             setting 2 (P2 fixed): dS1 = g P1 ((S1 - LSE1) - (S2 - LSE2) - KL)
//             and dQ_f = scale dS K_f, dK_f = scale dS^T Q_f for the free side f.
//
// Design (MI355X-first; the pages' own kernels target NVIDIA parts and are prior art only):
//  * All contractions run on v_mfma_f32_32x32x16_bf16 (bf16 in, fp32 accumulate), one wave64
//    per 32x32 output tile.
//  * The forward and the dQ kernel are query-major: a wave keeps the B operand fragments of its
//    32 query rows of Q1 and Q2 in registers for the whole kernel and computes S^T = K Q^T, so
//    each lane owns one query row and 16 of the keys of every 32-key block. Each lane then keeps
//    its own partial online state (m1, l1, m2, l2, acc) with no cross-lane traffic in the hot
//    loop; the two lanes that share a query merge their states once at the end (the merge of
//    two partial states is associative). The P1-weighted logit difference is accumulated from
//    the unscaled dot products and scaled once at the end. The running maxima are raised only on
//    a lane's first tile and on masked tiles; an overflowed wave is recomputed exactly.
//  * The dK kernel is key-major: a wave keeps its 32 key rows of K1 and K2 in registers and
//    computes S = Q K^T, so dS^T comes out of the accumulator already in the A-operand layout
//    of dK = dS^T Q. Symmetrically, the dQ kernel's dS is the A operand of dQ = dS K. The other
//    operand of each gradient product is read by columns from the streamed tile with the
//    transposing LDS read. The two backward kernels recompute S independently and never use
//    atomics: results are deterministic.
//  * Streamed tiles are loaded from HBM through buffer resources (scalar base and byte range per
//    stage, 32-bit per-thread offsets); the range check pads the ragged end with zero rows. The
//    forward stages its key tiles through registers into double-buffered LDS with rows padded by
//    16 bytes, so the 16 rows read by one 16-byte operand load fall in distinct banks. The
//    backward kernels load their tiles straight into three LDS stages (buffer loads that write
//    LDS), rows unpadded with their 16-byte chunks permuted so that both the row reads and the
//    transposing reads are free of bank conflicts. Every operand address is a register plus an
//    immediate.
//  * exp and log use the hardware base-2 instructions; scale * log2(e) is folded into one FMA
//    per element and the saved LSEs stay in natural-log units.
//  * Causal (top-left) masking skips whole tiles past the frontier; only tiles that straddle
//    the diagonal or the ragged end of a sequence take the masked path. Causal grids run the
//    longest row blocks first, and block ids are mapped so that the blocks resident on an XCD
//    are consecutive row blocks of one (batch, head) slice and share its tiles in L2.
//  * The dK kernel folds the upstream gradient into the exponents (g P = sign(g) 2^(y + log2|g|))
//    and applies the sign only on tiles that hold a negative g.
//  * Few query rows: a split-K forward (one wavefront per 32-row query block and key range up
//    to 32 rows, one block of the LDS-staged forward kernel per 256-row query block and key
//    range above; partial states merged by a lane group per row), a dQ kernel split over key
//    ranges with a deterministic sum of the partials, and a fused backward (n_q <= 64) that
//    forms dS once per key group and uses it for dK and for a per-block partial dQ, reading the
//    keys once; all three take a workspace from the caller.
//  * The forward is also built for fp8 e4m3 inputs (v_mfma_scale_f32_32x32x64_f8f6f4, one
//    dequantisation factor per side), with the same float32 state.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <type_traits>

#include "../../include/streamkl.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1.0e30f;  // finite stand-in for -inf in running maxima
constexpr float kInf = __builtin_huge_valf();

struct Shape {
  int nq, nk, bh, heads;
  long long q_sb, q_sh, q_sr;
  long long k_sb, k_sh, k_sr;
  float scale;
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// Waits until every global load of the wave has returned (s_waitcnt vmcnt(0); the expcnt and
// lgkmcnt fields are left at their maxima, i.e. not waited on). Called once after the loads of
// operands that stay in registers for a whole kernel: the compiler's wait placement merges a
// loop's entry and back edges, and without this it keeps waiting, inside the loop, for those
// long-finished loads by counting down the in-order load counter, which also waits for the
// next tile's prefetch and so cuts its lead to a few hundred cycles.
__device__ __forceinline__ void wait_global_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// The flag unchanged, passed through a VGPR so that the compiler takes it for a per-lane value.
// Used for the choice between the masked and unmasked dS variants in the backward kernels: when
// the compiler can see that the choice is wave-uniform (non-causal instances), it lays the two
// variants out so that their registers are live together and those instances spill; as a per-lane
// condition (as in the causal instances) they fit. At run time the flag is uniform either way.
__device__ __forceinline__ bool lane_flag(bool f) {
  int v = f;
  asm volatile("" : "+v"(v));
  return v != 0;
}

// Row (within a 32-row block) of accumulator register r of a 32x32 MFMA result for a lane in
// half h (lanes 32..63 are h = 1). The lane's column is lane & 31.
__device__ __forceinline__ int acc_row(int r, int h) { return (r >> 2) * 8 + h * 4 + (r & 3); }

__device__ __forceinline__ bf16x8 load_frag(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

// Eight fp32 values -> bf16x8 (round to nearest even).
__device__ __forceinline__ bf16x8 pack8(const float* v) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = static_cast<__bf16>(v[i]);
  return r;
}

// ---------------------------------------------------------------- LDS tiles
// A tile of ROWS rows x D bf16 values is stored row-major with a pitch of D + 8 elements: the
// 16-byte pad shifts consecutive rows by four banks, so the 16 rows that one pass of a 16-byte
// operand read touches fall in distinct banks, and every operand address of a lane is one base
// register plus a compile-time offset.
template <int D>
constexpr int lds_pitch() { return D + 8; }

// Streamed tiles are read through buffer resources (a scalar base address and a byte range):
// a load is the scalar base plus the thread's 32-bit offset plus a scalar offset, with no
// 64-bit address arithmetic per load, and the hardware's range check returns 0 for every byte
// past the range, which pads the ragged end of a matrix with zero rows without a per-row test.
// Row strides are kept below kMaxRowStrideBytes so that the offsets within a staged block of
// up to 128 rows fit in 32 bits (the C ABI rejects larger ones).
constexpr long long kMaxRowStrideBytes = 1LL << 24;
constexpr int kBufferWord3 = 0x00020000;  // 32-bit data format, no swizzle, raw addressing

// Resource for `rows` rows (clamped to [0, MAXR], MAXR <= 128) of rstride bytes from p.
template <int MAXR>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int rows,
                                                            long long rstride) {
  static_assert(MAXR <= 128, "MAXR rows of a stride below kMaxRowStrideBytes fit in 31 bits");
  int m = rows < MAXR ? rows : MAXR;
  // pinned to a scalar register between the two clamps: otherwise the pair is fused into a
  // vector median instruction, and the result has to be moved back to a scalar register
  asm volatile("" : "+s"(m));
  const int n = m > 0 ? m : 0;
  // uniform by construction; readfirstlane keeps the range in a scalar register (a resource in
  // vector registers would make every load a loop over the lanes' distinct values)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0,
                                           __builtin_amdgcn_readfirstlane(n * (int)rstride),
                                           kBufferWord3);
}

// Loads 16 bytes at offset voff + soff of the resource. On gfx950 the range check covers the
// whole offset (vector, scalar and instruction parts) dword by dword: a dword at or past the
// range reads as 0 (checked with a probe against a resource shorter than its allocation).
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, unsigned voff,
                                               unsigned soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Registers that stage ROWS rows of ROWB bytes from global memory into an LDS tile with a
// pitch of ROWB + 16 bytes (the forward's key tiles, any element format).
template <int ROWS, int ROWB, int NT>
struct TileRegs {
  static constexpr int CPR = ROWB / 16;  // 16-byte chunks per row
  static constexpr int N = (ROWS * CPR + NT - 1) / NT;
  static constexpr bool EVEN = N * NT == ROWS * CPR;  // else threads past the tile idle
  static_assert(NT % CPR == 0 && ROWS <= 128, "thread t: chunk t % CPR of rows t / CPR + k NT / CPR");
  uint4 v[N];

  // Rows row0.. of a [n_valid, ROWB bytes] matrix with a row stride of rstride bytes
  // (< kMaxRowStrideBytes); rows >= n_valid read as 0.
  __device__ __forceinline__ void load(const uint8_t* __restrict__ base, long long rstride,
                                       int row0, int n_valid) {
    const __amdgpu_buffer_rsrc_t r =
        make_rsrc<ROWS>(base + (long long)row0 * rstride, n_valid - row0, rstride);
    const unsigned off = (threadIdx.x / CPR) * (unsigned)rstride + (threadIdx.x % CPR) * 16u;
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (EVEN || threadIdx.x + i * NT < ROWS * CPR)
        v[i] = buffer_load16(r, off + (unsigned)(i * (NT / CPR)) * (unsigned)rstride, 0u);
  }
  __device__ __forceinline__ void store(uint8_t* lds) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = threadIdx.x + i * NT;
      const int row = idx / CPR, c = idx % CPR;
      if (EVEN || idx < ROWS * CPR) *reinterpret_cast<uint4*>(lds + row * (ROWB + 16) + c * 16) = v[i];
    }
  }
};

// A operand of a 32x32x16 MFMA: row `row` of the LDS tile, 8 values at columns
// kk * 16 + h * 8 .. +8.
template <int D>
__device__ __forceinline__ bf16x8 lds_a_frag(const uint16_t* lds, int row, int kk, int h) {
  return load_frag(lds + row * lds_pitch<D>() + kk * 16 + h * 8);
}

// ---------------------------------------------------------------- block -> tile mapping
// The hardware deals block ids round-robin to the 8 XCDs (id % 8), each with its own L2. The
// blocks of one slice stream the same tiles of the other side at about the same time, so they
// should share an XCD and be resident together.
// Interleaved mapping (any slice count): id = rank * n_slices + slice; with n_slices a multiple
// of 8 every block of a slice lands on the XCD of that slice, but the resident blocks of an XCD
// are a few ranks of several slices.
__device__ __forceinline__ void block_coords(int id, int n_slices, int& rank, int& slice) {
  rank = id / n_slices;
  slice = id - rank * n_slices;
}
// Grid of n_slices x (gridDim.x / n_slices) blocks: with n_slices a multiple of 8, XCD x runs the
// slices x, x + 8, ... one after another, their ranks in order, so the blocks resident on an
// XCD are consecutive ranks of one slice and share its tiles in L2 (64K causal, 32 heads:
// forward, dQ and dK each 2-3 % faster than the interleaved mapping). Otherwise interleaved.
__device__ __forceinline__ void block_coords(int n_slices, int& rank, int& slice) {
  if (n_slices % 8 != 0) {
    block_coords(blockIdx.x, n_slices, rank, slice);
    return;
  }
  const int nranks = gridDim.x / n_slices;
  const int id = blockIdx.x, xcd = id & 7, j = id >> 3;
  const int local = j / nranks;  // which of the XCD's slices
  rank = j - local * nranks;
  slice = xcd + 8 * local;
}

// ================================================================ forward
// Input formats of the forward's contractions. bf16: v_mfma_f32_32x32x16_bf16, 16 contraction
// elements per instruction. fp8: OCP e4m3 through v_mfma_scale_f32_32x32x64_f8f6f4 with unit
// (E8M0 = 127) block scales, 64 contraction elements per instruction. In both, a lane of the
// A (B) operand holds row (column) lane % 32 and the contraction elements
// (lane / 32) * KPER / 2 .. + KPER / 2 of the k-step in consecutive bytes, so one lane's operand
// is a contiguous piece of one row of a row-major tile.
typedef int i32x8 __attribute__((ext_vector_type(8)));

struct Bf16In {
  using Frag = bf16x8;
  static constexpr int EB = 2, KPER = 16;
  static __device__ __forceinline__ Frag load(const uint8_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
  }
  static __device__ __forceinline__ f32x16 mma(Frag a, Frag b, f32x16 c) { return mfma(a, b, c); }
};

struct Fp8In {
  using Frag = i32x8;
  static constexpr int EB = 1, KPER = 64;
  static __device__ __forceinline__ Frag load(const uint8_t* p) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint4 v = *reinterpret_cast<const uint4*>(p + 16);
    return Frag{(int)u.x, (int)u.y, (int)u.z, (int)u.w, (int)v.x, (int)v.y, (int)v.z, (int)v.w};
  }
  static __device__ __forceinline__ f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  }
};

// Each lane keeps its running state as a running maximum m_t (of the unscaled dot products x_t)
// and NP interleaved partial sums of l1, l2 and acc, all relative to exp2(c_t m_t) with
// c_t = scale * sigma_t * log2(e) (sigma_t = 1 for bf16 inputs, the dequantisation factor of
// side t for fp8 inputs): l_t = sum_j exp2(c_t (x_tj - m_t)) and
// acc = sum_j exp2(c_1 (x1j - m1)) (r12 x1j - x2j) with r12 = sigma_1 / sigma_2, so that the
// logit difference S1 - S2 = scale * sigma_2 * (r12 x1 - x2) costs one FMA.
//
// The running maximum is raised only where it must be: on a lane's first tile, and on tiles that
// take the masked path (the diagonal or the ragged end). Every other tile is accumulated against
// the current maximum without looking for a new one. That is the same sum up to rounding as long
// as no exponential overflows (fp32 keeps its relative precision up to 2^127), and it removes the
// tile maximum, the rescaling and the per-tile reduction from the common path. A lane whose state
// becomes non-finite, which needs a logit that exceeds every logit of its first tile by more than
// about 2^7 / c, is recomputed by the exact path at the end of the kernel.

// Adds one tile's exponentials to the partial sums against the current maxima (-c m_t = nb_t).
// s1 / s2 hold the lane's unscaled dot products of the tile: RB blocks of 32 keys, 16 keys of
// each block per lane. Masked entries are -inf and contribute 0.
template <int RB, bool MASK, int NP>
__device__ __forceinline__ void fwd_tile_accumulate(const f32x16 (&s1)[RB], const f32x16 (&s2)[RB],
                                                    float c1, float c2, float r12, float nb1,
                                                    float nb2, float (&L1)[NP], float (&L2)[NP],
                                                    float (&A)[NP]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float x1 = s1[rb][r], x2 = s2[rb][r];
      const float p1 = exp2_hw(fmaf(x1, c1, nb1));
      const float p2 = exp2_hw(fmaf(x2, c2, nb2));
      // masked entries have x1 = x2 = -inf and p1 = 0; their difference must not turn into NaN
      const float d12 = fmaf(x1, r12, -x2);
      const float dd = MASK ? (p1 > 0.f ? d12 : 0.f) : d12;
      const int j = r % NP;
      L1[j] += p1;
      L2[j] += p2;
      A[j] = fmaf(p1, dd, A[j]);
    }
  }
}

// One tile with the running maxima raised to the tile's maxima first (the partial sums are
// rescaled by exp2(c (m_old - m_new))). Applies the causal / ragged-end mask in place when MASK.
template <int RB, bool CAUSAL, bool MASK, int NP>
__device__ __forceinline__ void fwd_tile_exact(f32x16 (&s1)[RB], f32x16 (&s2)[RB], float c1,
                                               float c2, float r12, int key0, int query, int nk,
                                               int h, float& m1, float& m2, float& nb1, float& nb2,
                                               float (&L1)[NP], float (&L2)[NP], float (&A)[NP]) {
  if (MASK) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + rb * 32 + acc_row(r, h);
        const bool ok = key < nk && (!CAUSAL || key <= query);
        s1[rb][r] = ok ? s1[rb][r] : -kInf;
        s2[rb][r] = ok ? s2[rb][r] : -kInf;
      }
  }
  float mx1 = m1, mx2 = m2;
#pragma unroll
  for (int i = 0; i < 16 * RB; i += 2) {
    const int rb = i / 16, r = i % 16;
    mx1 = fmaxf(fmaxf(mx1, s1[rb][r]), s1[rb][r + 1]);
    mx2 = fmaxf(fmaxf(mx2, s2[rb][r]), s2[rb][r + 1]);
  }
  const float a1 = exp2_hw((m1 - mx1) * c1), a2 = exp2_hw((m2 - mx2) * c2);
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    L1[j] *= a1;
    L2[j] *= a2;
    A[j] *= a1;
  }
  m1 = mx1;
  m2 = mx2;
  nb1 = -mx1 * c1;
  nb2 = -mx2 * c2;
  fwd_tile_accumulate<RB, MASK, NP>(s1, s2, c1, c2, r12, nb1, nb2, L1, L2, A);
}

__device__ __forceinline__ bool non_finite(float x) {
  // bit test: stays valid when the compiler is told that NaNs do not occur
  return (__float_as_uint(x) & 0x7f800000u) == 0x7f800000u;
}

// Forward launch shape: blocks of kFwdWaves waves (32 query rows each), kFwdBlocksPerCU blocks
// resident per CU, key tiles of 32 * kFwdRB rows, LDS stages of fwd_stage_keys rows
// (double-buffered, one barrier per stage). The softmax-style update is VALU-bound and a single
// wave issues VALU instructions at a fraction of the SIMD's rate, so the shape favours several
// resident waves per SIMD.
constexpr int kFwdWaves = 8;
constexpr int kFwdBlocksPerCU = 1;
constexpr int kFwdRB = 1;
constexpr int kFwdThreads = 64 * kFwdWaves;
// Keys per stage. Without the causal mask 128-key stages (half the barriers) are faster (d = 64:
// -4.5 %, d = 128: -2 % at the non-causal workloads); with it the waves of a block leave the
// stage loop at different tiles near the diagonal and the larger stages cost more than the
// barriers they save (64K causal: +1.6 %), and 32-key stages cost +8 %.
template <bool CAUSAL>
constexpr int fwd_stage_keys() { return CAUSAL ? 64 : 128; }

// F: input format (Bf16In or Fp8In). q*/k* point at elements of that format; strides in the
// Shape are in elements. Side t's logits are scale * sigma_t * Q_t K_t^T.
// SPLIT (bf16 only): every block covers one key range of split_keys keys (a multiple of the
// stage) as well as one query block, and writes the partial state of its rows (M1, l1, M2, l2,
// acc, as the split-K kernel below does) to part [slice][range][5][n_q] instead of the outputs;
// fwd_merge_kernel finishes them.
template <class F, int D, bool CAUSAL, bool SHARED_K, bool SPLIT = false>
__global__ void __launch_bounds__(kFwdThreads, kFwdBlocksPerCU)
fwd_kernel(const uint8_t* __restrict__ q1, const uint8_t* __restrict__ k1,
           const uint8_t* __restrict__ q2, const uint8_t* __restrict__ k2,
           float* __restrict__ kl_out, float* __restrict__ lse1_out,
           float* __restrict__ lse2_out, Shape s, float sigma1, float sigma2,
           float* __restrict__ part = nullptr, int nsplit = 1, int split_keys = 0) {
  constexpr int EB = F::EB, KPER = F::KPER, KS = D / KPER;
  constexpr int RB = kFwdRB, BK = 32 * RB, SB = fwd_stage_keys<CAUSAL>(), BQ = 32 * kFwdWaves;
  constexpr int NKT = SHARED_K ? 1 : 2;
  static_assert(SB % BK == 0, "a stage holds whole tiles");
  static_assert(!SPLIT || std::is_same<F, Bf16In>::value, "key ranges: bf16 inputs");
  constexpr int ROWB = D * EB, PB = ROWB + 16, TILE = SB * PB;  // bytes
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * NKT * TILE];

  // block id = (range * query blocks + rank) * slices + slice: every block of a slice, whatever
  // its range, lands on the same XCD
  int rank, slice;
  block_coords(s.bh, rank, slice);
  const int nqb = (s.nq + BQ - 1) / BQ;
  int split = 0;
  if (SPLIT) {
    split = rank / nqb;
    rank -= split * nqb;
  }
  const int qb = CAUSAL ? nqb - 1 - rank : rank;
  const int b = slice / s.heads, hd = slice - b * s.heads;
  const uint8_t* Q1 = q1 + (b * s.q_sb + hd * s.q_sh) * EB;
  const uint8_t* Q2 = q2 + (b * s.q_sb + hd * s.q_sh) * EB;
  const uint8_t* K1 = k1 + (b * s.k_sb + hd * s.k_sh) * EB;
  const uint8_t* K2 = k2 + (b * s.k_sb + hd * s.k_sh) * EB;
  const long long qrs = s.q_sr * EB, krs = s.k_sr * EB;  // row strides in bytes

  const int l = lane_id(), w = wave_id(), h = l >> 5, col = l & 31;
  const int qw0 = qb * BQ + w * 32;
  const int query = qw0 + col;
  const int qrow = query < s.nq ? query : s.nq - 1;
  // byte offset of this lane's operand within a k-step of a row
  const int lane_off = h * (KPER / 2) * EB;

  typename F::Frag f1[KS], f2[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    f1[kk] = F::load(Q1 + qrow * qrs + kk * KPER * EB + lane_off);
    f2[kk] = F::load(Q2 + qrow * qrs + kk * KPER * EB + lane_off);
  }

  const int last_q = min(s.nq - 1, qb * BQ + BQ - 1);
  const int kvis = CAUSAL ? min(s.nk, last_q + 1) : s.nk;
  // keys [kbeg, kend) of this block; tile t starts at key kbeg + t BK
  const int kbeg = SPLIT ? split * split_keys : 0;
  const int kend = SPLIT ? min(kvis, kbeg + split_keys) : kvis;
  const int nkeys = kend > kbeg ? kend - kbeg : 0;
  const int ntiles = (nkeys + BK - 1) / BK;
  const int nstages = (nkeys + SB - 1) / SB;
  const uint8_t* K1r = K1 + (long long)kbeg * krs;
  const uint8_t* K2r = K2 + (long long)kbeg * krs;
  const int nk_r = s.nk - kbeg;  // rows of the key matrices from kbeg on
  const float c1 = s.scale * sigma1 * kLog2e, c2 = s.scale * sigma2 * kLog2e;
  const float r12 = sigma1 / sigma2;
  const bool wave_live = qw0 < s.nq;

  constexpr int NP = 4;  // interleaved partial sums per quantity
  float m1 = kNegBig, m2 = kNegBig, nb1 = 0.f, nb2 = 0.f;
  float L1[NP] = {}, L2[NP] = {}, A[NP] = {};
  TileRegs<SB, ROWB, kFwdThreads> r1, r2;
  r1.load(K1r, krs, 0, nk_r);
  if (!SHARED_K) r2.load(K2r, krs, 0, nk_r);
  r1.store(lds);
  if (!SHARED_K) r2.store(lds + TILE);
  if (nstages > 1) {
    r1.load(K1r, krs, SB, nk_r);
    if (!SHARED_K) r2.load(K2r, krs, SB, nk_r);
  }
  __syncthreads();

  f32x16 s1[RB], s2[RB];
  // S^T of the tile starting at row `row0` of the stage: 2 * RB independent accumulation chains
  auto contract = [&](const uint8_t* kt1, const uint8_t* kt2, int row0) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      s1[rb] = f32x16{};
      s2[rb] = f32x16{};
    }
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      typename F::Frag a1[RB], a2[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int off = (row0 + rb * 32 + col) * PB + kk * KPER * EB + lane_off;
        a1[rb] = F::load(kt1 + off);
        if (!SHARED_K) a2[rb] = F::load(kt2 + off);
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        s1[rb] = F::mma(a1[rb], f1[kk], s1[rb]);
        s2[rb] = F::mma(SHARED_K ? a1[rb] : a2[rb], f2[kk], s2[rb]);
      }
    }
  };

  for (int st = 0; st < nstages; ++st) {
    const uint8_t* kt1 = lds + (st & 1) * NKT * TILE;
    const uint8_t* kt2 = kt1 + (NKT - 1) * TILE;
#pragma unroll
    for (int sub = 0; sub < SB / BK; ++sub) {
      const int t = st * (SB / BK) + sub;
      const int key0 = kbeg + t * BK;
      // a tile is skipped when it is past the end or every key of it is past this wave's rows
      if (t < ntiles && wave_live && !(CAUSAL && key0 > qw0 + 31)) {
        contract(kt1, kt2, sub * BK);
        const bool full = (key0 + BK <= s.nk) && (!CAUSAL || key0 + BK - 1 <= qw0);
        if (full && t > 0)
          fwd_tile_accumulate<RB, false, NP>(s1, s2, c1, c2, r12, nb1, nb2, L1, L2, A);
        else if (full)
          fwd_tile_exact<RB, CAUSAL, false, NP>(s1, s2, c1, c2, r12, key0, query, s.nk, h, m1, m2,
                                                nb1, nb2, L1, L2, A);
        else
          fwd_tile_exact<RB, CAUSAL, true, NP>(s1, s2, c1, c2, r12, key0, query, s.nk, h, m1, m2,
                                               nb1, nb2, L1, L2, A);
      }
    }
    if (st + 1 < nstages) {
      // the other buffer was last read in stage st - 1, before the previous barrier
      uint8_t* nxt = lds + ((st + 1) & 1) * NKT * TILE;
      r1.store(nxt);
      if (!SHARED_K) r2.store(nxt + TILE);
      if (st + 2 < nstages) {
        r1.load(K1r, krs, (st + 2) * SB, nk_r);
        if (!SHARED_K) r2.load(K2r, krs, (st + 2) * SB, nk_r);
      }
    }
    __syncthreads();
  }

  float l1 = (L1[0] + L1[1]) + (L1[2] + L1[3]);
  float l2 = (L2[0] + L2[1]) + (L2[2] + L2[3]);
  float acc = (A[0] + A[1]) + (A[2] + A[3]);

  // Exact path for a wave with an overflowed lane: every tile again, each one raising the
  // maxima, with the key tiles read straight from global memory (no LDS, no barrier).
  const bool bad = non_finite(l1) || non_finite(l2) || non_finite(acc);
  if (wave_live && __any(bad)) {
    m1 = m2 = kNegBig;
#pragma unroll
    for (int j = 0; j < NP; ++j) L1[j] = L2[j] = A[j] = 0.f;
    const int wend = CAUSAL ? min(kend, qw0 + 32) : kend;
    for (int key0 = kbeg; key0 < wend; key0 += 32) {
      f32x16 x1[1] = {f32x16{}}, x2[1] = {f32x16{}};
      const long long ro = (long long)min(key0 + col, s.nk - 1) * krs + lane_off;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        x1[0] = F::mma(F::load(K1 + ro + kk * KPER * EB), f1[kk], x1[0]);
        x2[0] = F::mma(F::load(K2 + ro + kk * KPER * EB), f2[kk], x2[0]);
      }
      fwd_tile_exact<1, CAUSAL, true, NP>(x1, x2, c1, c2, r12, key0, query, s.nk, h, m1, m2, nb1,
                                          nb2, L1, L2, A);
    }
    l1 = (L1[0] + L1[1]) + (L1[2] + L1[3]);
    l2 = (L2[0] + L2[1]) + (L2[2] + L2[3]);
    acc = (A[0] + A[1]) + (A[2] + A[3]);
  }

  // Merge the two partial states of this query row (lanes l and l ^ 32).
  const float om1 = __shfl_xor(m1, 32), ol1 = __shfl_xor(l1, 32);
  const float om2 = __shfl_xor(m2, 32), ol2 = __shfl_xor(l2, 32);
  const float oacc = __shfl_xor(acc, 32);
  if (h == 0 && query < s.nq) {
    const float M1 = fmaxf(m1, om1), M2 = fmaxf(m2, om2);
    const float fa = exp2_hw((m1 - M1) * c1), fb = exp2_hw((om1 - M1) * c1);
    const float ga = exp2_hw((m2 - M2) * c2), gb = exp2_hw((om2 - M2) * c2);
    const float L1s = l1 * fa + ol1 * fb;
    const float L2s = l2 * ga + ol2 * gb;
    const float As = acc * fa + oacc * fb;
    if constexpr (SPLIT) {
      float* o = part + ((long long)slice * nsplit + split) * 5 * s.nq + query;
      o[0] = M1;
      o[s.nq] = L1s;
      o[2 * s.nq] = M2;
      o[3 * s.nq] = L2s;
      o[4 * s.nq] = As;
    } else {
      const float lse1 = M1 * (s.scale * sigma1) + log2_hw(L1s) * kLn2;
      const float lse2 = M2 * (s.scale * sigma2) + log2_hw(L2s) * kLn2;
      const long long o = (long long)slice * s.nq + query;
      kl_out[o] = (s.scale * sigma2) * As / L1s + (lse2 - lse1);
      lse1_out[o] = lse1;
      lse2_out[o] = lse2;
    }
  }
}

// ================================================================ split-K forward
// With few query rows (decode-like shapes) one block per 256-row query block leaves most of the
// chip idle. Here (up to 32 query rows; above, the key ranges run on fwd_kernel with SPLIT)
// every wave has its own work item: a 32-row query block of one slice and one contiguous range
// of key tiles. The wave reads its keys straight from global memory into MFMA
// operands (no LDS and no barrier: no other wave of the block reads the same keys), runs the
// forward's online update and writes the partial state of each row (m1, l1, m2, l2, acc; l and
// acc relative to exp2(c m)) to a workspace laid out [slice][range][5][n_q]. A second kernel
// merges the ranges of each row (merging two online states is associative: the larger maximum
// wins and the other sums are rescaled by exp2(c (m_a - m))) and finishes KL, LSE1 and LSE2.
constexpr int kSplitWaves = 4;  // independent work items per block

template <int D, bool CAUSAL, bool SHARED_K>
__global__ void __launch_bounds__(64 * kSplitWaves)
fwd_split_kernel(const uint16_t* __restrict__ q1, const uint16_t* __restrict__ k1,
                 const uint16_t* __restrict__ q2, const uint16_t* __restrict__ k2,
                 float* __restrict__ part, Shape s, int nsplit, int split_keys) {
  constexpr int KS = D / 16;
  const int nqb = (s.nq + 31) / 32;
  const long long item = (long long)blockIdx.x * kSplitWaves + wave_id();
  if (item >= (long long)s.bh * nqb * nsplit) return;  // nothing below synchronises the block
  const int split = (int)(item % nsplit);
  const long long rest = item / nsplit;
  const int qb = (int)(rest % nqb), slice = (int)(rest / nqb);
  const int b = slice / s.heads, hd = slice - b * s.heads;
  const uint16_t* Q1 = q1 + b * s.q_sb + hd * s.q_sh;
  const uint16_t* Q2 = q2 + b * s.q_sb + hd * s.q_sh;
  const uint16_t* K1 = k1 + b * s.k_sb + hd * s.k_sh;
  const uint16_t* K2 = k2 + b * s.k_sb + hd * s.k_sh;

  const int l = lane_id(), h = l >> 5, col = l & 31;
  const int q0 = qb * 32;
  const int query = q0 + col;
  const int qrow = query < s.nq ? query : s.nq - 1;
  bf16x8 f1[KS], f2[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    f1[kk] = load_frag(Q1 + (long long)qrow * s.q_sr + kk * 16 + h * 8);
    f2[kk] = load_frag(Q2 + (long long)qrow * s.q_sr + kk * 16 + h * 8);
  }
  const int kbeg = split * split_keys;
  int kend = min(s.nk, kbeg + split_keys);
  if (CAUSAL) kend = min(kend, min(s.nq - 1, q0 + 31) + 1);
  const float c = s.scale * kLog2e;

  float m1, m2, nb1, nb2, L1[4], L2[4], A[4];
  f32x16 x1[1], x2[1];
  // pass 0 raises the maxima only on the range's first tile and on masked tiles; a wave with a
  // lane whose state overflowed repeats its range with every tile raising them (pass 1)
  for (int pass = 0; pass < 2; ++pass) {
    m1 = m2 = kNegBig;
    nb1 = nb2 = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) L1[j] = L2[j] = A[j] = 0.f;
    // operands of the next tile are loaded while the current one is contracted and updated;
    // rows past n_k are read clamped and masked by the exact update
    bf16x8 a1[KS], a2[KS];
    auto fetch = [&](int key0) {
      const long long ro = (long long)min(key0 + col, s.nk - 1) * s.k_sr + h * 8;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        a1[kk] = load_frag(K1 + ro + kk * 16);
        if (!SHARED_K) a2[kk] = load_frag(K2 + ro + kk * 16);
      }
    };
    if (kbeg < kend) fetch(kbeg);
    for (int key0 = kbeg; key0 < kend; key0 += 32) {
      x1[0] = f32x16{};
      x2[0] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        x1[0] = mfma(a1[kk], f1[kk], x1[0]);
        x2[0] = mfma(SHARED_K ? a1[kk] : a2[kk], f2[kk], x2[0]);
      }
      if (key0 + 32 < kend) fetch(key0 + 32);
      const bool full = (key0 + 32 <= s.nk) && (!CAUSAL || key0 + 31 <= q0);
      if (pass == 0 && full && key0 > kbeg)
        fwd_tile_accumulate<1, false, 4>(x1, x2, c, c, 1.f, nb1, nb2, L1, L2, A);
      else if (full)
        fwd_tile_exact<1, CAUSAL, false, 4>(x1, x2, c, c, 1.f, key0, query, s.nk, h, m1, m2, nb1,
                                            nb2, L1, L2, A);
      else
        fwd_tile_exact<1, CAUSAL, true, 4>(x1, x2, c, c, 1.f, key0, query, s.nk, h, m1, m2, nb1,
                                           nb2, L1, L2, A);
    }
    const bool bad = non_finite((L1[0] + L1[1]) + (L1[2] + L1[3])) ||
                     non_finite((L2[0] + L2[1]) + (L2[2] + L2[3])) ||
                     non_finite((A[0] + A[1]) + (A[2] + A[3]));
    if (!__any(bad)) break;
  }
  float l1 = (L1[0] + L1[1]) + (L1[2] + L1[3]);
  float l2 = (L2[0] + L2[1]) + (L2[2] + L2[3]);
  float acc = (A[0] + A[1]) + (A[2] + A[3]);
  // merge the two halves of each row (lanes l and l ^ 32)
  const float om1 = __shfl_xor(m1, 32), ol1 = __shfl_xor(l1, 32);
  const float om2 = __shfl_xor(m2, 32), ol2 = __shfl_xor(l2, 32);
  const float oacc = __shfl_xor(acc, 32);
  if (h == 0 && query < s.nq) {
    const float M1 = fmaxf(m1, om1), M2 = fmaxf(m2, om2);
    const float fa = exp2_hw((m1 - M1) * c), fb = exp2_hw((om1 - M1) * c);
    const float ga = exp2_hw((m2 - M2) * c), gb = exp2_hw((om2 - M2) * c);
    float* o = part + ((long long)slice * nsplit + split) * 5 * s.nq + query;
    o[0] = M1;
    o[s.nq] = l1 * fa + ol1 * fb;
    o[2 * s.nq] = M2;
    o[3 * s.nq] = l2 * ga + ol2 * gb;
    o[4 * s.nq] = acc * fa + oacc * fb;
  }
}

// Merges the partial state (m, l) of one side and the side-1-weighted acc of another range
// into the running one (running maxima; c converts a logit difference to a base-2 exponent).
__device__ __forceinline__ void merge_partial(float& M1, float& L1, float& A, float& M2, float& L2,
                                              float m1, float l1, float a, float m2, float l2,
                                              float c) {
  const float n1 = fmaxf(M1, m1), n2 = fmaxf(M2, m2);
  const float fa = exp2_hw((M1 - n1) * c), fb = exp2_hw((m1 - n1) * c);
  const float ga = exp2_hw((M2 - n2) * c), gb = exp2_hw((m2 - n2) * c);
  L1 = fmaf(L1, fa, l1 * fb);
  A = fmaf(A, fa, a * fb);
  L2 = fmaf(L2, ga, l2 * gb);
  M1 = n1;
  M2 = n2;
}

// Merge of the nsplit partial states of each (slice, query row) and the row's outputs. A group of
// `group` lanes (a power of two up to 64, inside one wavefront) serves one row: lane j merges
// ranges j, j + group, ... in one pass, then the group combines its lanes' states by butterfly
// exchanges. With few rows and many ranges the ranges are read in parallel instead of by one
// thread in sequence.
__global__ void __launch_bounds__(256)
fwd_merge_kernel(const float* __restrict__ part, float* __restrict__ kl_out,
                 float* __restrict__ lse1_out, float* __restrict__ lse2_out, Shape s, int nsplit,
                 int group) {
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const int lane = (int)(gid & (group - 1));
  const long long idx = gid / group;
  const long long rows = (long long)s.bh * s.nq;
  // lanes of a row past the end still take part in the exchanges, on row 0, and write nothing
  const long long row = idx < rows ? idx : 0;
  const int slice = (int)(row / s.nq), q = (int)(row - (long long)slice * s.nq);
  const float c = s.scale * kLog2e;
  const float* p = part + (long long)slice * nsplit * 5 * s.nq + q;
  float M1 = kNegBig, M2 = kNegBig, L1 = 0.f, L2 = 0.f, A = 0.f;
  for (int i = lane; i < nsplit; i += group) {
    const float* pi = p + (long long)(5 * i) * s.nq;
    merge_partial(M1, L1, A, M2, L2, pi[0], pi[s.nq], pi[4 * s.nq], pi[2 * s.nq], pi[3 * s.nq], c);
  }
  for (int off = 1; off < group; off <<= 1) {
    const float m1 = __shfl_xor(M1, off), l1 = __shfl_xor(L1, off), a = __shfl_xor(A, off);
    const float m2 = __shfl_xor(M2, off), l2 = __shfl_xor(L2, off);
    merge_partial(M1, L1, A, M2, L2, m1, l1, a, m2, l2, c);
  }
  if (idx >= rows || lane != 0) return;
  const float lse1 = M1 * s.scale + log2_hw(L1) * kLn2;
  const float lse2 = M2 * s.scale + log2_hw(L2) * kLn2;
  kl_out[idx] = s.scale * A / L1 + (lse2 - lse1);
  lse1_out[idx] = lse1;
  lse2_out[idx] = lse2;
}

// ================================================================ backward
// Both backward kernels stream 32-row tiles of the "other" side (key rows for the dQ kernel,
// query rows for the dK kernel) through three LDS stages, one barrier per tile, with 8 waves of
// 32 stationary rows each. The S recomputation reads a streamed tile's rows (contraction over
// head_dim); the gradient product reads the free side's tile by columns (contraction over the
// streamed rows), in the order in which a 32x32 accumulator holds rows (acc_row), which makes
// the accumulator of dS directly the A operand of that product.
constexpr int kBwdWaves = 8;
constexpr int kBwdThreads = 64 * kBwdWaves;
constexpr int kBwdBlocksPerCU = 8 / kBwdWaves;  // 2 waves per SIMD
constexpr int kBT = 32;                          // streamed rows per tile

// Transposed copies (the fused backward's query rows and keys): row r of a 32-row block is
// stored at column tpos(r) (bits 2 and 3 of r swapped), so that lane half h of a 32x32x16 MFMA
// reads its eight rows 16c + {4h..4h+3, 8+4h..8+4h+3} as one contiguous 16-byte chunk.
constexpr int kTPitch = kBT + 8;  // pitch (elements) of a transposed block

__device__ __forceinline__ int tpos(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// B operand of a gradient product from a transposed block: rows (head_dim) nb*32 + (l & 31), the
// eight streamed rows of chunk cc for lane half h.
__device__ __forceinline__ bf16x8 tr_frag(const uint16_t* tr, int nb, int cc, int col, int h) {
  return load_frag(tr + (nb * 32 + col) * kTPitch + cc * 16 + h * 8);
}

// ---------------------------------------------------------------- streamed tiles, direct to LDS
// The backward kernels stream 32-row tiles of the other side's bf16 matrices. A tile goes from
// global memory straight into LDS (buffer loads with an LDS destination: no registers and no LDS
// store instructions), three stages deep: the loads of tile i + 2 are issued at the end of tile
// i and land while tile i + 1 is computed. Rows
// are unpadded (2 D bytes) and the 16-byte chunk c of row r sits at chunk position
// c ^ bwd_swz(r). The permutation keeps both operand reads free of LDS bank conflicts: the 16-byte
// row reads of the S recomputation (16 consecutive rows at one chunk per pass) and the 8-byte
// transposing reads (ds_read_b64_tr_b16; per 32 lanes four consecutive rows by four chunks) that
// give the gradient product its operand, columns of the row-major tile, with no transposed copy.
template <int D>
__device__ __forceinline__ int bwd_swz(int r) {
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// LDS byte address (as M0 and the DS instructions take it) of a pointer into a __shared__ array.
__device__ __forceinline__ unsigned lds_address(const void* p) {
  return (unsigned)(size_t)(const __attribute__((address_space(3))) void*)p;
}

// 16 bytes per lane from byte offset voff of resource r to LDS byte address lds + 16 * lane (a
// buffer load with an LDS destination; M0 holds the wave's LDS address, one wait state before
// the load reads it, and is restored afterwards: the compiler reserves M0 and does not expect
// inline assembly to change it). Written as inline assembly so that the compiler does not track
// it as an LDS write: it would wait for every such load before any later LDS read, the loads of
// stages prefetched for later tiles included. The kernels wait for these loads themselves
// (vmcnt) before the barrier that publishes a stage; the loads write no registers.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned lds) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(r), "s"(lds)
      : "memory");
}

// Waits until at most `keep` (0, 1 or 2; wave-uniform) vector memory loads of the wave are in
// flight (s_waitcnt vmcnt; expcnt and lgkmcnt not waited on), then keeps the compiler from moving
// memory accesses above the wait.
__device__ __forceinline__ void wait_loads_keep(int keep) {
  if (keep >= 2)
    __builtin_amdgcn_s_waitcnt(0x0F72);
  else if (keep == 1)
    __builtin_amdgcn_s_waitcnt(0x0F71);
  else
    __builtin_amdgcn_s_waitcnt(0x0F70);
  asm volatile("" ::: "memory");
}

// Direct-to-LDS staging of the NTENS streamed tensors of one tile: each tensor's tile is cut into
// 1 KB pieces (4 rows at d = 128), piece i loaded by wave i % 8.
template <int D, int NTENS>
struct BwdDma {
  static constexpr int TB = 32 * 2 * D;        // bytes of one tensor's tile
  static constexpr int PPT = TB / 1024;        // pieces per tensor
  static constexpr int PIECES = NTENS * PPT;
  static constexpr int N = (PIECES + kBwdWaves - 1) / kBwdWaves;  // loads per wave, at most
  static_assert(N <= 2, "wait_loads_keep covers two loads per wave and stage");
  static constexpr int STAGE = NTENS * TB;     // bytes of one stage
  unsigned voff[N];  // the lane's byte offset, from the tile's first row, for each load
  int cnt;           // the wave's loads per tile (wave-uniform)

  __device__ __forceinline__ void init(long long rstride_bytes) {
    const int w = __builtin_amdgcn_readfirstlane(wave_id()), l = lane_id();
    cnt = 0;
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int idx = w + j * kBwdWaves;
      const int o = (idx % PPT) * 1024 + 16 * l;  // byte of the lane's 16 bytes in the tile
      const int row = o / (2 * D), c = ((o % (2 * D)) / 16) ^ bwd_swz<D>(row);
      voff[j] = (unsigned)row * (unsigned)rstride_bytes + 16u * (unsigned)c;
      cnt += idx < PIECES ? 1 : 0;
    }
  }
  // Rows row0 .. row0 + 31 of two [n_valid, D] matrices (row stride rstride elements) into the
  // stage at LDS byte address `stage`; rows >= n_valid read as 0.
  __device__ __forceinline__ void issue(const uint16_t* __restrict__ b0,
                                        const uint16_t* __restrict__ b1, long long rstride,
                                        int row0, int n_valid, unsigned stage) const {
    const __amdgpu_buffer_rsrc_t r0 =
        make_rsrc<kBT>(b0 + (long long)row0 * rstride, n_valid - row0, rstride * 2);
    const __amdgpu_buffer_rsrc_t r1 =
        NTENS == 2 ? make_rsrc<kBT>(b1 + (long long)row0 * rstride, n_valid - row0, rstride * 2)
                   : r0;
    const int w = __builtin_amdgcn_readfirstlane(wave_id());
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int idx = w + j * kBwdWaves;
      if (PIECES % kBwdWaves == 0 || idx < PIECES) {
        const int te = idx / PPT;
        lds_dma16(te == 0 ? r0 : r1, voff[j], stage + (unsigned)(te * TB + (idx % PPT) * 1024));
      }
    }
  }
  // Waits for this wave's loads of every stage but the `pending` (0 or 1) issued last.
  __device__ __forceinline__ void wait(int pending) const { wait_loads_keep(pending * cnt); }
};

// A operand of the S recomputation from a swizzled tile: row `row` (0..31), head_dim values
// kk * 16 + h * 8 .. + 7. a_base = row * 2D + 16 * (h ^ bwd_swz(row)); the chunk's position is
// then a_base ^ 32 kk (the XOR touches only the bits below the row's).
__device__ __forceinline__ bf16x8 swz_a_frag(const unsigned char* tile, int a_base, int kk) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(tile + (a_base ^ (32 * kk))));
}

// Per-lane byte offsets of the transposing reads (ds_read_b64_tr_b16). In each group of 16
// lanes, lane j receives element j % 4 of the 8 bytes read by lanes 4 e + j / 4 (e = 0..3) as
// its elements e. For the B operand of a gradient product (lane l: tile rows
// acc_row(8 cc + i, h), i = 0..7, at column nb * 32 + (l & 31)), lane (e = (l >> 2) & 3,
// m = l & 3) of group g reads row 8 r + 4 h + e (r = 0, 1 for elements 0..3 and 4..7) at
// columns 16 (g & 1) + 4 m .. + 3; tb[r] is that offset for cc = 0 and nb = 0, column block
// nb is at tb[r] ^ 64 nb and cc = 1 sixteen rows further.
template <int D>
__device__ __forceinline__ void tr_bases(int l, int (&tb)[2]) {
  const int h = l >> 5, e = (l >> 2) & 3, m = l & 3;
  const int low = 2 * ((l >> 4) & 1) + (m >> 1);
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int row = 8 * r + 4 * h + e;
    tb[r] = row * 2 * D + 8 * (m & 1) + 16 * (low ^ bwd_swz<D>(row));
  }
}

// B operand of a gradient product for column block nb, chunk cc; `tile` points at the tile's
// first row for cc = 0 and 16 rows further for cc = 1.
__device__ __forceinline__ bf16x8 swz_tr_frag(const unsigned char* tile, const int (&tb)[2], int nb) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(tile + (tb[0] ^ (64 * nb))));
  const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(tile + (tb[1] ^ (64 * nb))));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// ---------------------------------------------------------------- dQ (query-major)
// With SPLIT, the key tiles are cut into nsplit ranges of split_tiles tiles and block
// (query block, slice, range) writes its float32 partial dQ (already scaled by g * scale) to
// part[range][slice][n_q][D]; dq_reduce_kernel sums the ranges. For few query rows this gives
// the chip enough blocks; every partial is written (zeros for a range a block cannot see), so
// the sum is deterministic and needs no atomics.
template <int D, int SETTING, bool CAUSAL, bool SHARED_K, bool SPLIT = false>
__global__ void __launch_bounds__(kBwdThreads, kBwdBlocksPerCU)
dq_kernel(const uint16_t* __restrict__ q1, const uint16_t* __restrict__ k1,
          const uint16_t* __restrict__ q2, const uint16_t* __restrict__ k2,
          const float* __restrict__ lse1, const float* __restrict__ lse2,
          const float* __restrict__ klv, const float* __restrict__ gv,
          __bf16* __restrict__ dq_out, Shape s, float* __restrict__ part = nullptr,
          int nsplit = 1, int split_tiles = 0) {
  constexpr int BQ = 32 * kBwdWaves, KS = D / 16, NB = D / 32;
  constexpr int NTENS = SHARED_K ? 1 : 2;
  constexpr int FREE = SHARED_K ? 0 : 2 - SETTING;  // tensor index of K_free (side 2 for setting 1)
  using DM = BwdDma<D, NTENS>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[3 * DM::STAGE];
  __shared__ float gscale[kBwdWaves][32];

  int rank, slice;
  const int split = SPLIT ? (int)(blockIdx.x % nsplit) : 0;
  if (SPLIT)
    block_coords((int)(blockIdx.x / nsplit), s.bh, rank, slice);
  else
    block_coords(s.bh, rank, slice);
  const int nqb = (s.nq + BQ - 1) / BQ;
  const int qb = CAUSAL ? nqb - 1 - rank : rank;
  const int b = slice / s.heads, hd = slice - b * s.heads;
  const uint16_t* Q1 = q1 + b * s.q_sb + hd * s.q_sh;
  const uint16_t* Q2 = q2 + b * s.q_sb + hd * s.q_sh;
  const uint16_t* K1 = k1 + b * s.k_sb + hd * s.k_sh;
  const uint16_t* K2 = k2 + b * s.k_sb + hd * s.k_sh;

  const int l = lane_id(), w = wave_id(), h = l >> 5, col = l & 31;
  const int qw0 = qb * BQ + w * 32;
  const int query = qw0 + col;
  const int qrow = query < s.nq ? query : s.nq - 1;
  const long long ro = (long long)slice * s.nq + qrow;

  bf16x8 f1[KS], f2[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    f1[kk] = load_frag(Q1 + (long long)qrow * s.q_sr + kk * 16 + h * 8);
    f2[kk] = load_frag(Q2 + (long long)qrow * s.q_sr + kk * 16 + h * 8);
  }
  const float c = s.scale * kLog2e;
  const float b1 = -lse1[ro] * kLog2e;
  const float b2 = -lse2[ro] * kLog2e;                                   // setting 1
  const float cst = SETTING == 2 ? (lse2[ro] - lse1[ro]) - klv[ro] : 0.f;  // setting 2
  if (h == 0) gscale[w][col] = gv[ro] * s.scale;
  wait_global_loads();

  const int last_q = min(s.nq - 1, qb * BQ + BQ - 1);
  const int kend = CAUSAL ? min(s.nk, last_q + 1) : s.nk;
  // key tiles [t0, t1) of this block
  const int t0 = SPLIT ? split * split_tiles : 0;
  const int t1 = SPLIT ? min((kend + kBT - 1) / kBT, t0 + split_tiles) : (kend + kBT - 1) / kBT;
  const bool wave_live = qw0 < s.nq;

  f32x16 dq[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) dq[nb] = f32x16{};

  // per-lane offsets of the operand reads in a stage (S recomputation and transposing reads)
  const int a_base = col * 2 * D + 16 * (h ^ bwd_swz<D>(col));
  int tb[2];
  tr_bases<D>(l, tb);
  DM dma;
  dma.init(s.k_sr * 2);
  const unsigned lds0 = __builtin_amdgcn_readfirstlane(lds_address(lds));
  const int n = t1 - t0;
  if (n > 0) dma.issue(K1, K2, s.k_sr, t0 * kBT, s.nk, lds0);
  if (n > 1) dma.issue(K1, K2, s.k_sr, (t0 + 1) * kBT, s.nk, lds0 + DM::STAGE);
  dma.wait(n > 1 ? 1 : 0);
  __syncthreads();

  // one tile; the loop is unrolled three times so that the stage (i % 3) is a compile-time
  // constant and every operand read is a per-lane register plus an immediate offset
  auto tile = [&](int i, auto stgc) {
    constexpr int STG = decltype(stgc)::value;
    const int t = t0 + i;
    const unsigned char* stage = lds + STG * DM::STAGE;
    const unsigned char* kt1 = stage;
    const unsigned char* kt2 = stage + (NTENS - 1) * DM::TB;
    const unsigned char* ktr = stage + FREE * DM::TB;
    const int key0 = t * kBT;
    const bool skip = !wave_live || (CAUSAL && key0 > qw0 + 31);
    if (!skip) {
      // S^T of the tile's 32 keys: 2 independent accumulation chains
      f32x16 x1 = f32x16{}, x2 = f32x16{};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const bf16x8 a1 = swz_a_frag(kt1, a_base, kk);
        const bf16x8 a2 = SHARED_K ? a1 : swz_a_frag(kt2, a_base, kk);
        x1 = mfma(a1, f1[kk], x1);
        x2 = mfma(a2, f2[kk], x2);
      }
      // dS of the 32-key block and its dQ product; the element mask is compiled only into the
      // variant used on tiles that straddle the diagonal or the ragged end
      auto ds_block = [&](auto maskc) {
        constexpr bool MASK = decltype(maskc)::value;
        float ds[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float e1 = x1[r], e2 = x2[r];
          const float d12 = e1 - e2;
          if (MASK) {
            const int key = key0 + acc_row(r, h);
            const bool ok = key < s.nk && (!CAUSAL || key <= query);
            e1 = ok ? e1 : -kInf;
            e2 = ok ? e2 : -kInf;
          }
          const float p1 = exp2_hw(fmaf(e1, c, b1));
          if (SETTING == 1)
            ds[r] = exp2_hw(fmaf(e2, c, b2)) - p1;
          else
            ds[r] = p1 * fmaf(d12, s.scale, cst);
        }
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const bf16x8 a = pack8(ds + 8 * cc);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            dq[nb] = mfma(a, swz_tr_frag(ktr + cc * 32 * D, tb, nb), dq[nb]);
        }
      };
      if (lane_flag((key0 + 32 <= s.nk) && (!CAUSAL || key0 + 31 <= qw0)))
        ds_block(std::false_type{});
      else
        ds_block(std::true_type{});
    }
    // tile i + 2 into the stage tile i - 1 used (free since the last barrier), issued after this
    // tile's operand reads so that its LDS writes do not meet them
    if (i + 2 < n)
      dma.issue(K1, K2, s.k_sr, (t + 2) * kBT, s.nk, lds0 + ((STG + 2) % 3) * DM::STAGE);
    if (i + 1 < n) dma.wait(i + 2 < n ? 1 : 0);
    __syncthreads();
  };
  for (int i = 0; i < n;) {
    tile(i, std::integral_constant<int, 0>{});
    if (++i >= n) break;
    tile(i, std::integral_constant<int, 1>{});
    if (++i >= n) break;
    tile(i, std::integral_constant<int, 2>{});
    ++i;
  }
  if (!wave_live) return;
  const long long obase = (long long)slice * s.nq;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int qr = qw0 + acc_row(r, h);
    if (qr < s.nq) {
      const float gsc = gscale[w][acc_row(r, h)];
      if (SPLIT) {
        float* dst = part + (((long long)split * s.bh) * s.nq + obase + qr) * D + col;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) dst[nb * 32] = dq[nb][r] * gsc;
      } else {
        __bf16* dst = dq_out + (obase + qr) * D + col;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) dst[nb * 32] = static_cast<__bf16>(dq[nb][r] * gsc);
      }
    }
  }
}

// Sum of the nsplit float32 partials of dQ (part[range][rows * D]), rounded once to bfloat16;
// one thread per 4 consecutive elements.
__global__ void __launch_bounds__(256)
dq_reduce_kernel(const float* __restrict__ part, __bf16* __restrict__ dq, long long n4, int nsplit) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const float4* p = reinterpret_cast<const float4*>(part) + i;
  float4 a = p[0];
  for (int r = 1; r < nsplit; ++r) {
    const float4 v = p[(long long)r * n4];
    a.x += v.x;
    a.y += v.y;
    a.z += v.z;
    a.w += v.w;
  }
  const bf16x2 lo = {static_cast<__bf16>(a.x), static_cast<__bf16>(a.y)};
  const bf16x2 hi = {static_cast<__bf16>(a.z), static_cast<__bf16>(a.w)};
  reinterpret_cast<uint2*>(dq)[i] =
      make_uint2(__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi));
}

// ---------------------------------------------------------------- dK (key-major)
template <int D, int SETTING, bool CAUSAL, bool SHARED_K>
__global__ void __launch_bounds__(kBwdThreads, kBwdBlocksPerCU)
dk_kernel(const uint16_t* __restrict__ q1, const uint16_t* __restrict__ k1,
          const uint16_t* __restrict__ q2, const uint16_t* __restrict__ k2,
          const float* __restrict__ lse1, const float* __restrict__ lse2,
          const float* __restrict__ klv, const float* __restrict__ gv,
          __bf16* __restrict__ dk_out, Shape s) {
  constexpr int BKW = 32 * kBwdWaves, KS = D / 16, NB = D / 32;
  constexpr int FREE = 2 - SETTING;  // tensor index of Q_free (side 2 for setting 1)
  using DM = BwdDma<D, 2>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[3 * DM::STAGE];
  // Per stage, the constants wave 0 makes from the tile's per-query inputs: per query the
  // exponent bias of P1 and of P2 (setting 1) or LSE2 - LSE1 - KL (setting 2), with log2 |g|
  // folded into the exponent biases (g P = sign(g) 2^(y + log2 |g|)), and sign(g). Tiles whose g
  // are all >= 0 (flag qneg = 0) never read the sign.
  __shared__ __attribute__((aligned(16))) float qa[3][3][kBT];
  __shared__ int qneg[3];

  int rank, slice;
  block_coords(s.bh, rank, slice);
  const int kb = rank;  // causal: small kb sees the most queries, so it runs first
  const int b = slice / s.heads, hd = slice - b * s.heads;
  const uint16_t* Q1 = q1 + b * s.q_sb + hd * s.q_sh;
  const uint16_t* Q2 = q2 + b * s.q_sb + hd * s.q_sh;
  const uint16_t* K1 = k1 + b * s.k_sb + hd * s.k_sh;
  const uint16_t* K2 = k2 + b * s.k_sb + hd * s.k_sh;
  const long long rbase = (long long)slice * s.nq;

  const int l = lane_id(), w = wave_id(), h = l >> 5, col = l & 31;
  const int kw0 = kb * BKW + w * 32;
  const int key = kw0 + col;
  const int krow = key < s.nk ? key : s.nk - 1;

  bf16x8 f1[KS], f2[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    f1[kk] = load_frag(K1 + (long long)krow * s.k_sr + kk * 16 + h * 8);
    f2[kk] = SHARED_K ? f1[kk] : load_frag(K2 + (long long)krow * s.k_sr + kk * 16 + h * 8);
  }
  wait_global_loads();
  const float c = s.scale * kLog2e;
  // query tiles run from the last one down to the first visible one, so that the blocks of one
  // slice, which start together, stream the same tiles at the same time
  const int t_lo = CAUSAL ? (kb * BKW) / kBT : 0;
  const int t_hi = (s.nq + kBT - 1) / kBT - 1;
  const bool wave_live = kw0 < s.nk;

  f32x16 dk[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) dk[nb] = f32x16{};

  const int a_base = col * 2 * D + 16 * (h ^ bwd_swz<D>(col));
  int tb[2];
  tr_bases<D>(l, tb);
  DM dma;
  dma.init(s.q_sr * 2);
  const unsigned lds0 = __builtin_amdgcn_readfirstlane(lds_address(lds));
  // Per-query inputs of the next tile (wave 0, lanes 0..31, one query each), loaded into
  // registers a tile before they are turned into that tile's constants, so that nothing waits
  // for them in between.
  float rx1 = 0.f, rx2 = 0.f, rg = 0.f, rkl = 0.f;
  bool rvalid = false;
  auto load_inputs = [&](int t) {
    if (threadIdx.x < kBT) {
      const int q = t * kBT + threadIdx.x;
      rvalid = q < s.nq;
      if (rvalid) {
        rx1 = lse1[rbase + q];
        rx2 = lse2[rbase + q];
        rg = gv[rbase + q];
        if (SETTING == 2) rkl = klv[rbase + q];
      }
    }
  };
  auto make_constants = [&](int stg) {
    if (threadIdx.x < kBT) {
      // rows past n_q (and rows with g = 0) get P = 0: bias -inf
      float cq0 = -kInf, cq1 = SETTING == 1 ? -kInf : 0.f, cq2 = 1.f;
      if (rvalid) {
        const float lg = rg != 0.f ? log2_hw(fabsf(rg)) : -kInf;
        cq0 = fmaf(-rx1, kLog2e, lg);
        cq1 = SETTING == 1 ? fmaf(-rx2, kLog2e, lg) : (rx2 - rx1) - rkl;
        cq2 = rg < 0.f ? -1.f : 1.f;
      }
      const bool neg = __any(rvalid && rg < 0.f);
      qa[stg][0][threadIdx.x] = cq0;
      qa[stg][1][threadIdx.x] = cq1;
      qa[stg][2][threadIdx.x] = cq2;
      if (threadIdx.x == 0) qneg[stg] = neg ? 1 : 0;
    }
  };
  // Query tile t (Q1 and Q2 rows) into stage stg; rows past n_q read as 0. The compiler does not
  // see these loads (inline assembly), so its own wait for the per-query inputs (vmcnt 0) also
  // waits for them: the inputs are loaded after the tile and used a tile later, as the tile is.
  auto issue = [&](int t, int stg) {
    dma.issue(Q1, Q2, s.q_sr, t * kBT, s.nq, lds0 + stg * DM::STAGE);
  };
  const int n = t_hi >= t_lo ? t_hi - t_lo + 1 : 0;
  if (n > 0) issue(t_hi, 0);
  if (n > 1) issue(t_hi - 1, 1);
  if (n > 0) {
    load_inputs(t_hi);
    dma.wait(n > 1 ? 1 : 0);
    make_constants(0);
    if (n > 1) load_inputs(t_hi - 1);
  }
  __syncthreads();

  // one tile; the loop is unrolled three times so that the stage (i % 3) is a compile-time
  // constant and every operand read is a per-lane register plus an immediate offset
  auto tile = [&](int i, auto stgc) {
    constexpr int STG = decltype(stgc)::value;
    const int t = t_hi - i;
    const unsigned char* stage = lds + STG * DM::STAGE;
    const unsigned char* qt1 = stage;
    const unsigned char* qt2 = stage + DM::TB;
    const unsigned char* qtr = stage + FREE * DM::TB;
    const int qt0 = t * kBT;
    const bool skip = !wave_live || (CAUSAL && qt0 + kBT - 1 < kw0);
    if (!skip) {
      f32x16 x1 = f32x16{}, x2 = f32x16{};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        x1 = mfma(swz_a_frag(qt1, a_base, kk), f1[kk], x1);
        x2 = mfma(swz_a_frag(qt2, a_base, kk), f2[kk], x2);
      }
      // dS^T of the 32-query block and its dK product; the element mask is compiled only into
      // the variant used on tiles that straddle the diagonal or the ragged end
      auto ds_block = [&](auto maskc, auto signc) {
        constexpr bool MASK = decltype(maskc)::value;
        constexpr bool SIGNED = decltype(signc)::value;  // some g < 0 in this tile
        float ds[16];
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          // registers 4rq..4rq+3 hold 4 consecutive queries
          const int qi = rq * 8 + h * 4;
          const float4 va0 = *reinterpret_cast<const float4*>(&qa[STG][0][qi]);
          const float4 va1 = *reinterpret_cast<const float4*>(&qa[STG][1][qi]);
          const float4 va2 = SIGNED ? *reinterpret_cast<const float4*>(&qa[STG][2][qi])
                                    : make_float4(1.f, 1.f, 1.f, 1.f);
          const float c0[4] = {va0.x, va0.y, va0.z, va0.w};
          const float c1[4] = {va1.x, va1.y, va1.z, va1.w};
          const float c2[4] = {va2.x, va2.y, va2.z, va2.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = rq * 4 + j;
            float e1 = x1[r], e2 = x2[r];
            const float d12 = e1 - e2;
            if (MASK) {
              const int q = qt0 + qi + j;
              const bool ok = q < s.nq && (!CAUSAL || key <= q);
              e1 = ok ? e1 : -kInf;
              e2 = ok ? e2 : -kInf;
            }
            // g P1 and g P2 with |g| inside the exponent
            const float p1 = exp2_hw(fmaf(e1, c, c0[j]));
            float v;
            if (SETTING == 1)
              v = exp2_hw(fmaf(e2, c, c1[j])) - p1;
            else
              v = p1 * fmaf(d12, s.scale, c1[j]);
            ds[r] = SIGNED ? c2[j] * v : v;
          }
        }
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const bf16x8 a = pack8(ds + 8 * cc);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            dk[nb] = mfma(a, swz_tr_frag(qtr + cc * 32 * D, tb, nb), dk[nb]);
        }
      };
      const bool signed_tile = qneg[STG] != 0;
      const bool full = lane_flag((qt0 + 32 <= s.nq) && (!CAUSAL || qt0 >= kw0 + 31));
      // two variants only (a third costs registers): tiles that straddle the diagonal or the
      // ragged end, or hold a negative g, take the masked variant that applies the sign
      if (full && !signed_tile)
        ds_block(std::false_type{}, std::false_type{});
      else
        ds_block(std::true_type{}, std::true_type{});
    }
    if (i + 1 < n) {
      dma.wait(0);
      make_constants((STG + 1) % 3);
    }
    // tile i + 2 into the stage tile i - 1 used (free since the last barrier), issued after this
    // tile's operand reads so that its LDS writes do not meet them, and after the wait above
    if (i + 2 < n) {
      issue(t - 2, (STG + 2) % 3);
      load_inputs(t - 2);
    }
    __syncthreads();
  };
  for (int i = 0; i < n;) {
    tile(i, std::integral_constant<int, 0>{});
    if (++i >= n) break;
    tile(i, std::integral_constant<int, 1>{});
    if (++i >= n) break;
    tile(i, std::integral_constant<int, 2>{});
    ++i;
  }
  if (!wave_live) return;
  const long long obase = (long long)slice * s.nk;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int kr = kw0 + acc_row(r, h);
    if (kr < s.nk) {
      __bf16* dst = dk_out + (obase + kr) * D + col;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) dst[nb * 32] = static_cast<__bf16>(dk[nb][r] * s.scale);
    }
  }
}

// ---------------------------------------------------------------- fused backward (few queries)
// For few query rows one key-major pass gives dK of the free side and, from the same dS tiles,
// each key block's partial dQ, so that the keys are read once instead of once per gradient. All
// query rows stay in LDS (Q1 and Q2 row-major, the free side also transposed); each wave walks
// `groups` groups of 32 keys (a block covers groups * 128 consecutive keys, so that the staging of
// the query rows and the block's dQ partial are paid once per many keys). The dQ product needs
// dS with queries as rows, so each tile's dS goes
// through a per-wave LDS scratch, and the wave's free-side keys are kept transposed in LDS as
// that product's other operand. The block's partial dQ (already times scale) goes to
// part[key block][slice][n_q][D]; dq_reduce_kernel sums the key blocks in a fixed order.
constexpr int kFusedWaves = 4;  // one wave per SIMD: room for the dQ accumulators
constexpr int kFusedThreads = 64 * kFusedWaves;
constexpr int kFusedStep = 32 * kFusedWaves;  // keys of one step of the block's waves
constexpr int kFusedMaxGroups = 64;           // 32-key groups per wave, at most
constexpr int kFusedMaxQ = 64;                // query rows the fused path takes
constexpr int kDsPitch = 32 + 8;                             // pitch (elements) of the dS scratch

// Row `row` (columns col0..col0 + 7) of a tile into its transposed copy: element (row, col0 + j)
// goes to transposed row col0 + j at position `pos`, as 16-bit stores.
__device__ __forceinline__ void store_transposed8(uint16_t* tr, int pos, int col0, uint4 v) {
  const unsigned w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    tr[(col0 + 2 * j) * kTPitch + pos] = (uint16_t)(w4[j] & 0xFFFFu);
    tr[(col0 + 2 * j + 1) * kTPitch + pos] = (uint16_t)(w4[j] >> 16);
  }
}

// NQT: 32-row query tiles held (1 for n_q <= 32, else 2); fewer tiles, fewer registers and LDS.
template <int D, int SETTING, bool CAUSAL, bool SHARED_K, int NQT>
__global__ void __launch_bounds__(kFusedThreads, 1)
fused_bwd_kernel(const uint16_t* __restrict__ q1, const uint16_t* __restrict__ k1,
                 const uint16_t* __restrict__ q2, const uint16_t* __restrict__ k2,
                 const float* __restrict__ lse1, const float* __restrict__ lse2,
                 const float* __restrict__ klv, const float* __restrict__ gv,
                 __bf16* __restrict__ dk_out, float* __restrict__ part, Shape s, int groups) {
  constexpr int KS = D / 16, NB = D / 32, P = lds_pitch<D>(), CPR = D / 8;
  constexpr int MQ = 32 * NQT;  // query rows held
  constexpr int FREE = 2 - SETTING;  // tensor index of the free side (1 = side 2)
  __shared__ __attribute__((aligned(16))) uint16_t qrm[2][MQ * P];
  __shared__ __attribute__((aligned(16))) uint16_t qtr[NQT][D * kTPitch];
  __shared__ __attribute__((aligned(16))) uint16_t ktr[kFusedWaves][D * kTPitch];
  __shared__ __attribute__((aligned(16))) uint16_t dsq[kFusedWaves][32 * kDsPitch];
  __shared__ __attribute__((aligned(16))) float qa[3][MQ];
  __shared__ __attribute__((aligned(16))) float dqacc[MQ * D];
  __shared__ int qneg;

  int kb, slice;
  block_coords(s.bh, kb, slice);
  const int b = slice / s.heads, hd = slice - b * s.heads;
  const uint16_t* Q1 = q1 + b * s.q_sb + hd * s.q_sh;
  const uint16_t* Q2 = q2 + b * s.q_sb + hd * s.q_sh;
  const uint16_t* K1 = k1 + b * s.k_sb + hd * s.k_sh;
  const uint16_t* K2 = k2 + b * s.k_sb + hd * s.k_sh;
  const long long rbase = (long long)slice * s.nq;
  const int l = lane_id(), w = wave_id(), h = l >> 5, col = l & 31;
  const int nqt = (s.nq + 31) / 32;

  // every query row: Q1 and Q2 row-major (rows past n_q zero), the free side also transposed
  // (position tpos(row) of its 32-row tile, the order of a dS accumulator's rows)
  for (int idx = threadIdx.x; idx < 2 * MQ * CPR; idx += kFusedThreads) {
    const int te = idx / (MQ * CPR);
    const int rem = idx - te * (MQ * CPR);
    const int row = rem % MQ, chunk = rem / MQ;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (row < s.nq)
      v = *reinterpret_cast<const uint4*>((te ? Q2 : Q1) + row * s.q_sr + chunk * 8);
    *reinterpret_cast<uint4*>(&qrm[te][row * P + chunk * 8]) = v;
    if (te == FREE) store_transposed8(qtr[row / 32], tpos(row % 32), chunk * 8, v);
  }
  // per query: exponent biases with log2 |g| folded in and sign(g), as in the dK kernel
  if (threadIdx.x < MQ) {
    const int q = threadIdx.x;
    float cq0 = -kInf, cq1 = SETTING == 1 ? -kInf : 0.f, cq2 = 1.f;
    bool neg = false;
    if (q < s.nq) {
      const float x1 = lse1[rbase + q], x2 = lse2[rbase + q], g = gv[rbase + q];
      const float lg = g != 0.f ? log2_hw(fabsf(g)) : -kInf;
      cq0 = fmaf(-x1, kLog2e, lg);
      cq1 = SETTING == 1 ? fmaf(-x2, kLog2e, lg) : (x2 - x1) - klv[rbase + q];
      cq2 = g < 0.f ? -1.f : 1.f;
      neg = g < 0.f;
    }
    qa[0][q] = cq0;
    qa[1][q] = cq1;
    qa[2][q] = cq2;
    const bool any_neg = __any(neg);
    if (q == 0) qneg = any_neg ? 1 : 0;
  }
  __syncthreads();
  const bool signed_q = qneg != 0;
  const float c = s.scale * kLog2e;

  f32x16 pq[NQT][NB];  // this wave's partial dQ, queries as rows
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) pq[qt][nb] = f32x16{};

  // S operands of one 32-key group of this wave (rows past n_k read the last key; their dS is
  // masked)
  auto fetch = [&](int grp, bf16x8* a1, bf16x8* a2) {
    const int key = (kb * groups + grp) * kFusedStep + w * 32 + col;
    const long long ro = (long long)(key < s.nk ? key : s.nk - 1) * s.k_sr;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      a1[kk] = load_frag(K1 + ro + kk * 16 + h * 8);
      a2[kk] = SHARED_K ? a1[kk] : load_frag(K2 + ro + kk * 16 + h * 8);
    }
  };
  bf16x8 f1[KS], f2[KS];
  fetch(0, f1, f2);
  for (int grp = 0; grp < groups; ++grp) {
    const int kw0 = (kb * groups + grp) * kFusedStep + w * 32;
    if (kw0 >= s.nk) break;  // later groups lie further on
    const int key = kw0 + col;
    // the group's free-side keys transposed (head_dim as rows, keys in natural order), from
    // the S operands: lane (key, h) holds head_dim kk * 16 + h * 8 .. + 7 of step kk
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
      store_transposed8(ktr[w], col, kk * 16 + h * 8,
                        __builtin_bit_cast(uint4, FREE ? f2[kk] : f1[kk]));
    // with one query tile the next group's operands are fetched now (unconditionally, so that
    // the compiler counts the waits); with two there is no room for them and they are fetched
    // after the group
    bf16x8 n1[KS], n2[KS];
    if (NQT == 1) fetch(grp + 1 < groups ? grp + 1 : grp, n1, n2);
    const bool ragged = kw0 + 32 > s.nk;
    f32x16 dk[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) dk[nb] = f32x16{};
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      const int qt0 = qt * 32;
      if (qt >= nqt || (CAUSAL && qt0 + 31 < kw0)) continue;
      const uint16_t* qt1 = qrm[0] + qt0 * P;
      const uint16_t* qt2 = qrm[1] + qt0 * P;
      f32x16 x1 = f32x16{}, x2 = f32x16{};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        x1 = mfma(lds_a_frag<D>(qt1, col, kk, h), f1[kk], x1);
        x2 = mfma(lds_a_frag<D>(qt2, col, kk, h), f2[kk], x2);
      }
      // dS^T with g folded in (masked variant: queries past n_q, keys past n_k, the causal
      // diagonal, and the sign of g), its dK product, and dS stored with queries as rows
      auto ds_tile = [&](auto maskc) {
        constexpr bool MASK = decltype(maskc)::value;
        float ds[16];
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int qi = qt0 + rq * 8 + h * 4;
          const float4 va0 = *reinterpret_cast<const float4*>(&qa[0][qi]);
          const float4 va1 = *reinterpret_cast<const float4*>(&qa[1][qi]);
          const float4 va2 = MASK ? *reinterpret_cast<const float4*>(&qa[2][qi])
                                  : make_float4(1.f, 1.f, 1.f, 1.f);
          const float c0[4] = {va0.x, va0.y, va0.z, va0.w};
          const float c1[4] = {va1.x, va1.y, va1.z, va1.w};
          const float cs[4] = {va2.x, va2.y, va2.z, va2.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = rq * 4 + j;
            float e1 = x1[r], e2 = x2[r];
            const float d12 = e1 - e2;
            if (MASK) {
              const int q = qi + j;
              const bool ok = q < s.nq && key < s.nk && (!CAUSAL || key <= q);
              e1 = ok ? e1 : -kInf;
              e2 = ok ? e2 : -kInf;
            }
            const float p1 = exp2_hw(fmaf(e1, c, c0[j]));
            float v;
            if (SETTING == 1)
              v = exp2_hw(fmaf(e2, c, c1[j])) - p1;
            else
              v = p1 * fmaf(d12, s.scale, c1[j]);
            ds[r] = MASK ? cs[j] * v : v;
          }
        }
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const bf16x8 a = pack8(ds + 8 * cc);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            dk[nb] = mfma(a, tr_frag(qtr[qt], nb, cc, col, h), dk[nb]);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r)
          dsq[w][acc_row(r, h) * kDsPitch + col] =
              __builtin_bit_cast(uint16_t, static_cast<__bf16>(ds[r]));
      };
      if (lane_flag((qt0 + 32 <= s.nq) && !ragged && !signed_q && (!CAUSAL || qt0 >= kw0 + 31)))
        ds_tile(std::false_type{});
      else
        ds_tile(std::true_type{});
      // partial dQ of the tile over the group's keys: dS (queries as rows) times K_free
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const bf16x8 a = load_frag(&dsq[w][col * kDsPitch + cc * 16 + h * 8]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          pq[qt][nb] = mfma(a, tr_frag(ktr[w], nb, cc, col, h), pq[qt][nb]);
      }
    }
    // dK rows of the group's keys
    const long long obase = (long long)slice * s.nk;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = kw0 + acc_row(r, h);
      if (kr < s.nk) {
        __bf16* dst = dk_out + (obase + kr) * D + col;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) dst[nb * 32] = static_cast<__bf16>(dk[nb][r] * s.scale);
      }
    }
    if (NQT == 1) {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        f1[kk] = n1[kk];
        f2[kk] = n2[kk];
      }
    } else if (grp + 1 < groups) {
      fetch(grp + 1, f1, f2);
    }
  }
  // the block's partial dQ: the waves' accumulators summed in LDS in wave order (wave 0
  // stores, waves 1, 2, 3 add in turn, one barrier per turn), so the float32 sum has a fixed
  // order and the result is the same on every run; then written times scale
#pragma unroll
  for (int turn = 0; turn < kFusedWaves; ++turn) {
    if (w == turn) {
#pragma unroll
      for (int qt = 0; qt < NQT; ++qt) {
        if (qt >= nqt) continue;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float* a = &dqacc[(qt * 32 + acc_row(r, h)) * D + nb * 32 + col];
            *a = turn == 0 ? pq[qt][nb][r] : *a + pq[qt][nb][r];
          }
      }
    }
    __syncthreads();
  }
  float* dst = part + ((long long)kb * s.bh + slice) * s.nq * D;
  for (int i = threadIdx.x * 4; i < s.nq * D; i += kFusedThreads * 4) {
    float4 v = *reinterpret_cast<const float4*>(&dqacc[i]);
    v.x *= s.scale;
    v.y *= s.scale;
    v.z *= s.scale;
    v.w *= s.scale;
    *reinterpret_cast<float4*>(dst + i) = v;
  }
}

// ================================================================ host side
thread_local std::string g_last_error;

streamkl_status_t fail(streamkl_status_t st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

struct Span {
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

// Bytes from a [B, H, N, D] tensor's first element to one past its last, or -1 when that does
// not fit in 62 bits (no memory has such strides).
int64_t tensor_extent(int64_t B, int64_t H, int64_t N, int64_t D, const int64_t* st,
                      int64_t elem) {
  int64_t a, b, c, sum;
  if (__builtin_mul_overflow(B - 1, st[0], &a) || __builtin_mul_overflow(H - 1, st[1], &b) ||
      __builtin_mul_overflow(N - 1, st[2], &c) || __builtin_add_overflow(a, b, &sum) ||
      __builtin_add_overflow(sum, c, &sum) || __builtin_add_overflow(sum, D, &sum) ||
      __builtin_mul_overflow(sum, elem, &sum) || sum >= ((int64_t)1 << 62))
    return -1;
  return sum;
}

// Byte range of a tensor whose extent validate() has accepted.
Span tensor_span(const void* p, int64_t B, int64_t H, int64_t N, int64_t D, const int64_t* st,
                 int64_t elem) {
  const int64_t ext = tensor_extent(B, H, N, D, st, elem);
  return {reinterpret_cast<uintptr_t>(p), reinterpret_cast<uintptr_t>(p) + (uintptr_t)ext};
}

Span flat_span(const void* p, int64_t n, int64_t elem) {
  return {reinterpret_cast<uintptr_t>(p), reinterpret_cast<uintptr_t>(p) + (uintptr_t)(n * elem)};
}

streamkl_status_t validate(const streamkl_problem_t* p, const void* q1, const void* k1,
                           const void* q2, const void* k2, Shape* s, int elem_bytes = 2) {
  if (!p) return fail(STREAMKL_ERROR_INVALID_VALUE, "problem is NULL");
  if (p->batch < 1 || p->heads < 1 || p->n_q < 1 || p->n_k < 1)
    return fail(STREAMKL_ERROR_INVALID_VALUE, "batch, heads, n_q and n_k must be >= 1");
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(STREAMKL_ERROR_NOT_SUPPORTED, "head_dim must be 64 or 128");
  if (!(p->scale > 0.f) || !(p->scale < __builtin_huge_valf()))
    return fail(STREAMKL_ERROR_INVALID_VALUE, "scale must be finite and > 0");
  if (p->causal != 0 && p->causal != 1) return fail(STREAMKL_ERROR_INVALID_VALUE, "causal must be 0 or 1");
  const int64_t lim = (int64_t)1 << 30;
  // each factor is bounded before the product is formed (no signed overflow)
  if (p->batch >= lim || p->heads >= lim || p->n_q >= lim || p->n_k >= lim ||
      p->batch * p->heads >= lim)
    return fail(STREAMKL_ERROR_INVALID_VALUE, "sizes too large");
  const int64_t nblk = (p->n_q > p->n_k ? p->n_q : p->n_k) / 128 + 1;
  if (nblk * p->batch * p->heads >= ((int64_t)1 << 31))
    return fail(STREAMKL_ERROR_INVALID_VALUE, "grid too large");
  const int64_t sm = 16 / elem_bytes;  // strides keep every row 16-byte aligned
  for (int i = 0; i < 3; ++i) {
    if (p->q_stride[i] < 0 || p->k_stride[i] < 0 || p->q_stride[i] % sm || p->k_stride[i] % sm)
      return fail(STREAMKL_ERROR_INVALID_VALUE, "strides must be non-negative multiples of " +
                                                    std::to_string(sm) + " elements");
  }
  if (p->q_stride[2] < p->head_dim || p->k_stride[2] < p->head_dim)
    return fail(STREAMKL_ERROR_INVALID_VALUE, "row stride must be >= head_dim");
  if (p->q_stride[2] * elem_bytes >= kMaxRowStrideBytes ||
      p->k_stride[2] * elem_bytes >= kMaxRowStrideBytes)
    return fail(STREAMKL_ERROR_NOT_SUPPORTED, "row strides must be below 16 MiB");
  const int64_t qext = tensor_extent(p->batch, p->heads, p->n_q, p->head_dim, p->q_stride, elem_bytes);
  const int64_t kext = tensor_extent(p->batch, p->heads, p->n_k, p->head_dim, p->k_stride, elem_bytes);
  if (qext < 0 || kext < 0)
    return fail(STREAMKL_ERROR_INVALID_VALUE, "strides too large: a tensor's extent overflows");
  const void* in[4] = {q1, k1, q2, k2};
  const int64_t ext[4] = {qext, kext, qext, kext};
  for (int i = 0; i < 4; ++i) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(in[i]);
    if (!x) return fail(STREAMKL_ERROR_INVALID_VALUE, "input pointer is NULL");
    if (x % 16) return fail(STREAMKL_ERROR_INVALID_VALUE, "inputs must be 16-byte aligned");
    if (x > UINTPTR_MAX - (uintptr_t)ext[i])
      return fail(STREAMKL_ERROR_INVALID_VALUE, "an input's extent wraps the address space");
  }
  s->nq = (int)p->n_q;
  s->nk = (int)p->n_k;
  s->bh = (int)(p->batch * p->heads);
  s->heads = (int)p->heads;
  s->q_sb = p->q_stride[0];
  s->q_sh = p->q_stride[1];
  s->q_sr = p->q_stride[2];
  s->k_sb = p->k_stride[0];
  s->k_sh = p->k_stride[1];
  s->k_sr = p->k_stride[2];
  s->scale = p->scale;
  return STREAMKL_SUCCESS;
}

streamkl_status_t check_outputs(const streamkl_problem_t* p, const void* q1, const void* k1,
                                const void* q2, const void* k2, const Span* outs, int n_out,
                                const char* what, int elem_bytes = 2) {
  const Span in[4] = {
      tensor_span(q1, p->batch, p->heads, p->n_q, p->head_dim, p->q_stride, elem_bytes),
      tensor_span(k1, p->batch, p->heads, p->n_k, p->head_dim, p->k_stride, elem_bytes),
      tensor_span(q2, p->batch, p->heads, p->n_q, p->head_dim, p->q_stride, elem_bytes),
      tensor_span(k2, p->batch, p->heads, p->n_k, p->head_dim, p->k_stride, elem_bytes)};
  for (int i = 0; i < n_out; ++i) {
    if (outs[i].lo == 0) return fail(STREAMKL_ERROR_INVALID_VALUE, std::string(what) + ": output pointer is NULL");
    if (outs[i].lo % 16) return fail(STREAMKL_ERROR_INVALID_VALUE, std::string(what) + ": outputs must be 16-byte aligned");
    if (outs[i].hi < outs[i].lo)
      return fail(STREAMKL_ERROR_INVALID_VALUE, std::string(what) + ": an output's extent wraps the address space");
    for (const Span& x : in)
      if (overlaps(outs[i], x)) return fail(STREAMKL_ERROR_INVALID_VALUE, std::string(what) + ": output overlaps an input");
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], outs[j])) return fail(STREAMKL_ERROR_INVALID_VALUE, std::string(what) + ": outputs overlap");
  }
  return STREAMKL_SUCCESS;
}

streamkl_status_t check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(STREAMKL_ERROR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  g_last_error.clear();
  return STREAMKL_SUCCESS;
}

template <class F, int D, bool CAUSAL, bool SK>
void launch_fwd(const Shape& s, const void* q1, const void* k1, const void* q2, const void* k2,
                float* kl, float* l1, float* l2, float sigma1, float sigma2, hipStream_t st) {
  const int nqb = (s.nq + 32 * kFwdWaves - 1) / (32 * kFwdWaves);
  hipLaunchKernelGGL((fwd_kernel<F, D, CAUSAL, SK>), dim3(nqb * s.bh), dim3(kFwdThreads), 0, st,
                     (const uint8_t*)q1, (const uint8_t*)k1, (const uint8_t*)q2,
                     (const uint8_t*)k2, kl, l1, l2, s, sigma1, sigma2);
}

template <class F>
void dispatch_fwd(int64_t d, bool causal, bool sk, const Shape& s, const void* q1, const void* k1,
                  const void* q2, const void* k2, float* kl, float* l1, float* l2, float sigma1,
                  float sigma2, hipStream_t st) {
#define SKL_FWD(DD, C, S) launch_fwd<F, DD, C, S>(s, q1, k1, q2, k2, kl, l1, l2, sigma1, sigma2, st)
  if (d == 64) {
    if (causal) { if (sk) SKL_FWD(64, true, true); else SKL_FWD(64, true, false); }
    else { if (sk) SKL_FWD(64, false, true); else SKL_FWD(64, false, false); }
  } else {
    if (causal) { if (sk) SKL_FWD(128, true, true); else SKL_FWD(128, true, false); }
    else { if (sk) SKL_FWD(128, false, true); else SKL_FWD(128, false, false); }
  }
#undef SKL_FWD
}

// Key ranges of the split-K forward: n_splits requested (<= 0: chosen here) -> keys per range
// and the number of ranges actually used (no range is empty of key granules). With one 32-row
// query block per slice (n_q <= 32) every wave is a work item that reads its keys straight
// from global memory (granules of 32 keys); with more query rows those waves would each read
// the same keys again, so the work items are blocks of the LDS-staged forward kernel, one
// 256-row query block by one key range (granules of one stage: 64 keys causal, 128 without).
// (32 heads, 64K keys: the two paths take the same time at 24-32 rows; at 33-64 rows the blocks
// take 0.21 ms against 0.25-0.29 ms.)
constexpr int kSplitWaveMaxRows = 32;

struct SplitPlan {
  int nsplit, split_keys;
  bool blocks;  // ranges run on the LDS-staged forward kernel
};

SplitPlan split_plan(const streamkl_problem_t* p, int32_t n_splits) {
  const bool blocks = p->n_q > kSplitWaveMaxRows;
  const int64_t gran = blocks ? (p->causal ? fwd_stage_keys<true>() : fwd_stage_keys<false>()) : 32;
  // with the top-left causal mask no row sees a key past n_q - 1
  const int64_t nvis = p->causal && p->n_q < p->n_k ? p->n_q : p->n_k;
  const int64_t ngran = (nvis + gran - 1) / gran;
  const int64_t rows_per_item = blocks ? 32 * kFwdWaves : 32;
  const int64_t items = p->batch * p->heads * ((p->n_q + rows_per_item - 1) / rows_per_item);
  int64_t ns = n_splits;
  if (ns <= 0) {
    // wave items: about 1024 waves (one per SIMD; at 32 heads and 64K keys 1024 items ran 7 %
    // faster than 4096, with fewer partial states to merge); block items: about two blocks per
    // CU (one resident at a time). At least 8 granules per range; no split at all when there
    // are as many items as CUs already (the one-pass forward is then the better path).
    const int64_t target = blocks ? 512 : 1024;
    if (items > 256) {
      ns = 1;
    } else {
      ns = (target + items - 1) / items;
      const int64_t cap = (ngran + 7) / 8;
      if (ns > cap) ns = cap;
    }
  }
  if (ns > ngran) ns = ngran;
  if (ns > 4096) ns = 4096;
  if (ns < 1) ns = 1;
  const int64_t per = (ngran + ns - 1) / ns;
  const int64_t used = (ngran + per - 1) / per;
  return {(int)used, (int)(per * gran), blocks};
}

size_t split_workspace_bytes(const streamkl_problem_t* p, int nsplit) {
  return (size_t)p->batch * p->heads * p->n_q * nsplit * 5 * sizeof(float);
}

// Blocks launched by the split-K forward for this plan.
long long split_blocks(const Shape& s, const SplitPlan& plan) {
  if (plan.blocks)
    return (long long)s.bh * ((s.nq + 32 * kFwdWaves - 1) / (32 * kFwdWaves)) * plan.nsplit;
  const long long items = (long long)s.bh * ((s.nq + 31) / 32) * plan.nsplit;
  return (items + kSplitWaves - 1) / kSplitWaves;
}

template <int D, bool CAUSAL, bool SK>
void launch_fwd_split(const Shape& s, const SplitPlan& plan, const void* q1, const void* k1,
                      const void* q2, const void* k2, float* part, float* kl, float* l1,
                      float* l2, hipStream_t st) {
  const long long blocks = split_blocks(s, plan);
  if (plan.blocks)
    hipLaunchKernelGGL((fwd_kernel<Bf16In, D, CAUSAL, SK, true>), dim3((unsigned)blocks),
                       dim3(kFwdThreads), 0, st, (const uint8_t*)q1, (const uint8_t*)k1,
                       (const uint8_t*)q2, (const uint8_t*)k2, nullptr, nullptr, nullptr, s, 1.f,
                       1.f, part, plan.nsplit, plan.split_keys);
  else
    hipLaunchKernelGGL((fwd_split_kernel<D, CAUSAL, SK>), dim3((unsigned)blocks),
                       dim3(64 * kSplitWaves), 0, st, (const uint16_t*)q1, (const uint16_t*)k1,
                       (const uint16_t*)q2, (const uint16_t*)k2, part, s, plan.nsplit,
                       plan.split_keys);
  const long long rows = (long long)s.bh * s.nq;
  int group = 1;  // lanes per row in the merge: the ranges' count rounded up to a power of two
  while (group < 64 && group < plan.nsplit) group *= 2;
  const long long threads = rows * group;
  hipLaunchKernelGGL(fwd_merge_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st,
                     (const float*)part, kl, l1, l2, s, plan.nsplit, group);
}

template <int D, int SET, bool CAUSAL, bool SK>
void launch_bwd(const Shape& s, const void* q1, const void* k1, const void* q2, const void* k2,
                const float* l1, const float* l2, const float* kl, const float* g, void* dq,
                void* dk, hipStream_t st) {
  const int nqb = (s.nq + 32 * kBwdWaves - 1) / (32 * kBwdWaves);
  const int nkb = (s.nk + 32 * kBwdWaves - 1) / (32 * kBwdWaves);
  if (dq)
    hipLaunchKernelGGL((dq_kernel<D, SET, CAUSAL, SK>), dim3(nqb * s.bh), dim3(kBwdThreads), 0, st,
                       (const uint16_t*)q1, (const uint16_t*)k1, (const uint16_t*)q2,
                       (const uint16_t*)k2, l1, l2, kl, g, (__bf16*)dq, s);
  if (dk)
    hipLaunchKernelGGL((dk_kernel<D, SET, CAUSAL, SK>), dim3(nkb * s.bh), dim3(kBwdThreads), 0, st,
                       (const uint16_t*)q1, (const uint16_t*)k1, (const uint16_t*)q2,
                       (const uint16_t*)k2, l1, l2, kl, g, (__bf16*)dk, s);
}

// Key ranges of the split dQ kernel: ranges of whole 32-key tiles of the visible key span.
struct DqSplitPlan {
  int nsplit, split_tiles;
};

DqSplitPlan dq_split_plan(const streamkl_problem_t* p, int32_t n_splits) {
  const int64_t nvis = p->causal && p->n_q < p->n_k ? p->n_q : p->n_k;
  const int64_t ntiles = (nvis + kBT - 1) / kBT;
  const int64_t blocks = p->batch * p->heads * ((p->n_q + 32 * kBwdWaves - 1) / (32 * kBwdWaves));
  int64_t ns = n_splits;
  if (ns <= 0) {
    if (blocks >= 256) {
      ns = 1;  // the dQ kernel already has a block for every CU
    } else {
      // about one block per CU (at 32 heads and 64K keys 3-7 % faster than two), at least 16
      // key tiles per range
      ns = (256 + blocks - 1) / blocks;
      const int64_t cap = (ntiles + 15) / 16;
      if (ns > cap) ns = cap;
    }
  }
  if (ns > ntiles) ns = ntiles;
  if (ns > 1024) ns = 1024;
  if (ns < 1) ns = 1;
  const int64_t per = (ntiles + ns - 1) / ns;
  return {(int)((ntiles + per - 1) / per), (int)per};
}

size_t dq_split_workspace_bytes(const streamkl_problem_t* p, int nsplit) {
  return nsplit > 1 ? (size_t)nsplit * p->batch * p->heads * p->n_q * p->head_dim * sizeof(float)
                    : 0;
}

template <int D, int SET, bool CAUSAL, bool SK>
void launch_dq_split(const Shape& s, const DqSplitPlan& plan, const void* q1, const void* k1,
                     const void* q2, const void* k2, const float* l1, const float* l2,
                     const float* kl, const float* g, void* dq, float* part, hipStream_t st) {
  const int nqb = (s.nq + 32 * kBwdWaves - 1) / (32 * kBwdWaves);
  hipLaunchKernelGGL((dq_kernel<D, SET, CAUSAL, SK, true>), dim3(nqb * s.bh * plan.nsplit),
                     dim3(kBwdThreads), 0, st, (const uint16_t*)q1, (const uint16_t*)k1,
                     (const uint16_t*)q2, (const uint16_t*)k2, l1, l2, kl, g, (__bf16*)dq, s,
                     part, plan.nsplit, plan.split_tiles);
  const long long n4 = (long long)s.bh * s.nq * D / 4;
  hipLaunchKernelGGL(dq_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st,
                     (const float*)part, (__bf16*)dq, n4, plan.nsplit);
}

template <int SET>
void dispatch_dq_split(int64_t d, bool causal, bool sk, const Shape& s, const DqSplitPlan& plan,
                       const void* q1, const void* k1, const void* q2, const void* k2,
                       const float* l1, const float* l2, const float* kl, const float* g,
                       void* dq, float* part, hipStream_t st) {
#define SKL_DQS(DD, C, S) \
  launch_dq_split<DD, SET, C, S>(s, plan, q1, k1, q2, k2, l1, l2, kl, g, dq, part, st)
  if (d == 64) {
    if (causal) { if (sk) SKL_DQS(64, true, true); else SKL_DQS(64, true, false); }
    else { if (sk) SKL_DQS(64, false, true); else SKL_DQS(64, false, false); }
  } else {
    if (causal) { if (sk) SKL_DQS(128, true, true); else SKL_DQS(128, true, false); }
    else { if (sk) SKL_DQS(128, false, true); else SKL_DQS(128, false, false); }
  }
#undef SKL_DQS
}

template <int SET>
void dispatch_bwd(int64_t d, bool causal, bool sk, const Shape& s, const void* q1,
                  const void* k1, const void* q2, const void* k2, const float* l1,
                  const float* l2, const float* kl, const float* g, void* dq, void* dk,
                  hipStream_t st) {
#define SKL_BWD(DD, C, S) launch_bwd<DD, SET, C, S>(s, q1, k1, q2, k2, l1, l2, kl, g, dq, dk, st)
  if (d == 64) {
    if (causal) { if (sk) SKL_BWD(64, true, true); else SKL_BWD(64, true, false); }
    else { if (sk) SKL_BWD(64, false, true); else SKL_BWD(64, false, false); }
  } else {
    if (causal) { if (sk) SKL_BWD(128, true, true); else SKL_BWD(128, true, false); }
    else { if (sk) SKL_BWD(128, false, true); else SKL_BWD(128, false, false); }
  }
#undef SKL_BWD
}

// Key groups per wave of the fused backward: as many as keep about one block per CU (256
// blocks; at 32 heads and 64K keys 5-7 % faster than two per CU, with half the workspace),
// between 1 and kFusedMaxGroups.
int fused_groups(const streamkl_problem_t* p) {
  const int64_t steps = (p->n_k + kFusedStep - 1) / kFusedStep;  // per slice
  int64_t g = steps * p->batch * p->heads / 256;
  if (g > kFusedMaxGroups) g = kFusedMaxGroups;
  if (g > steps) g = steps;
  return g < 1 ? 1 : (int)g;
}

int64_t fused_key_blocks(const streamkl_problem_t* p) {
  const int64_t keys = (int64_t)kFusedStep * fused_groups(p);
  return (p->n_k + keys - 1) / keys;
}

size_t fused_workspace_bytes(const streamkl_problem_t* p) {
  return (size_t)fused_key_blocks(p) * p->batch * p->heads * p->n_q * p->head_dim * sizeof(float);
}

template <int D, int SET, bool CAUSAL, bool SK>
void launch_fused(const Shape& s, int groups, const void* q1, const void* k1, const void* q2,
                  const void* k2, const float* l1, const float* l2, const float* kl,
                  const float* g, void* dq, void* dk, float* part, hipStream_t st) {
  const int nkb = (s.nk + kFusedStep * groups - 1) / (kFusedStep * groups);
  if (s.nq <= 32)
    hipLaunchKernelGGL((fused_bwd_kernel<D, SET, CAUSAL, SK, 1>), dim3(nkb * s.bh),
                       dim3(kFusedThreads), 0, st, (const uint16_t*)q1, (const uint16_t*)k1,
                       (const uint16_t*)q2, (const uint16_t*)k2, l1, l2, kl, g, (__bf16*)dk,
                       part, s, groups);
  else
    hipLaunchKernelGGL((fused_bwd_kernel<D, SET, CAUSAL, SK, 2>), dim3(nkb * s.bh),
                       dim3(kFusedThreads), 0, st, (const uint16_t*)q1, (const uint16_t*)k1,
                       (const uint16_t*)q2, (const uint16_t*)k2, l1, l2, kl, g, (__bf16*)dk,
                       part, s, groups);
  const long long n4 = (long long)s.bh * s.nq * D / 4;
  hipLaunchKernelGGL(dq_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st,
                     (const float*)part, (__bf16*)dq, n4, nkb);
}

template <int SET>
void dispatch_fused(int64_t d, bool causal, bool sk, const Shape& s, int groups, const void* q1,
                    const void* k1, const void* q2, const void* k2, const float* l1,
                    const float* l2, const float* kl, const float* g, void* dq, void* dk,
                    float* part, hipStream_t st) {
#define SKL_FUS(DD, C, S) \
  launch_fused<DD, SET, C, S>(s, groups, q1, k1, q2, k2, l1, l2, kl, g, dq, dk, part, st)
  if (d == 64) {
    if (causal) { if (sk) SKL_FUS(64, true, true); else SKL_FUS(64, true, false); }
    else { if (sk) SKL_FUS(64, false, true); else SKL_FUS(64, false, false); }
  } else {
    if (causal) { if (sk) SKL_FUS(128, true, true); else SKL_FUS(128, true, false); }
    else { if (sk) SKL_FUS(128, false, true); else SKL_FUS(128, false, false); }
  }
#undef SKL_FUS
}

// Which kernels a backward call runs.
enum class BwdPath {
  kSeparate,  // dq_kernel + dk_kernel (no workspace)
  kSplitDq,   // dq_kernel over key ranges + dq_reduce_kernel, and dk_kernel
  kFused,     // fused_bwd_kernel + dq_reduce_kernel (n_q <= kFusedMaxQ)
};

struct BwdPlan {
  BwdPath path;
  DqSplitPlan dq;  // key ranges of the dQ kernel (kSplitDq)
  size_t workspace;
};

// The adaptive choice of the plain backward entry points, from the problem's sizes alone.
// With few query rows the keys dominate the traffic and one key-major pass that forms dS once
// for both gradients is fastest (the fused path: 1.6-1.7x the split pair at n_q <= 64, 32 heads,
// 64K keys); above that, while the one-kernel dQ has fewer than 256 blocks, its keys are split
// into ranges; otherwise the two one-kernel passes, which need no workspace.
BwdPlan bwd_auto_plan(const streamkl_problem_t* p) {
  if (p->n_q <= kFusedMaxQ) return {BwdPath::kFused, {1, 0}, fused_workspace_bytes(p)};
  const DqSplitPlan dq = dq_split_plan(p, 0);
  if (dq.nsplit > 1) return {BwdPath::kSplitDq, dq, dq_split_workspace_bytes(p, dq.nsplit)};
  return {BwdPath::kSeparate, {1, 0}, 0};
}

// How the caller chose the kernels: the adaptive plan, one gradient's one-kernel pass, the key
// split dQ with a requested range count, or the fused pass.
enum class BwdMode { kAuto, kOneKernel, kSplitDq, kFused };

streamkl_status_t bwd_common(const streamkl_problem_t* p, int setting, const void* q1,
                             const void* k1, const void* q2, const void* k2, const float* lse1,
                             const float* lse2, const float* kl, const float* grad_kl, void* dq,
                             void* dk, bool want_dq, bool want_dk, hipStream_t stream,
                             const char* what, BwdMode mode, int32_t dq_splits = 0,
                             void* workspace = nullptr, size_t workspace_bytes = 0) {
  Shape s;
  streamkl_status_t st = validate(p, q1, k1, q2, k2, &s);
  if (st != STREAMKL_SUCCESS) return st;
  if (setting != 1 && setting != 2) return fail(STREAMKL_ERROR_INVALID_VALUE, std::string(what) + ": setting must be 1 or 2");
  if (!lse1 || !lse2 || !grad_kl || (setting == 2 && !kl))
    return fail(STREAMKL_ERROR_INVALID_VALUE, std::string(what) + ": NULL lse / kl / grad pointer");
  const int64_t n = p->batch * p->heads * p->n_q;
  if (mode == BwdMode::kFused && p->n_q > kFusedMaxQ)
    return fail(STREAMKL_ERROR_NOT_SUPPORTED,
                std::string(what) + ": n_q must be at most " + std::to_string(kFusedMaxQ));
  BwdPlan plan = {BwdPath::kSeparate, {1, 0}, 0};
  if (mode == BwdMode::kAuto) {
    plan = bwd_auto_plan(p);
  } else if (mode == BwdMode::kFused) {
    plan = {BwdPath::kFused, {1, 0}, fused_workspace_bytes(p)};
  } else if (mode == BwdMode::kSplitDq) {
    const DqSplitPlan dq = dq_split_plan(p, dq_splits);
    if (dq.nsplit > 1) plan = {BwdPath::kSplitDq, dq, dq_split_workspace_bytes(p, dq.nsplit)};
  }
  const size_t need = plan.workspace;
  if (workspace_bytes < need)
    return fail(STREAMKL_ERROR_INVALID_VALUE,
                std::string(what) + ": workspace too small (" + std::to_string(workspace_bytes) +
                    " < " + std::to_string(need) + " bytes)");
  Span outs[3];
  int n_out = 0;
  if (want_dq) outs[n_out++] = flat_span(dq, n * p->head_dim, 2);
  if (want_dk) outs[n_out++] = flat_span(dk, p->batch * p->heads * p->n_k * p->head_dim, 2);
  if (need > 0) outs[n_out++] = flat_span(workspace, (int64_t)need, 1);
  st = check_outputs(p, q1, k1, q2, k2, outs, n_out, what);
  if (st != STREAMKL_SUCCESS) return st;
  const Span vin[4] = {flat_span(lse1, n, 4), flat_span(lse2, n, 4), flat_span(grad_kl, n, 4),
                       flat_span(setting == 2 ? kl : lse1, n, 4)};
  for (int i = 0; i < n_out; ++i)
    for (const Span& v : vin)
      if (overlaps(outs[i], v)) return fail(STREAMKL_ERROR_INVALID_VALUE, std::string(what) + ": output overlaps an input");
  if (plan.path == BwdPath::kSplitDq &&
      (int64_t)plan.dq.nsplit * p->batch * p->heads * ((p->n_q + 255) / 256) >= ((int64_t)1 << 31))
    return fail(STREAMKL_ERROR_INVALID_VALUE, std::string(what) + ": grid too large");
  if (plan.path == BwdPath::kFused && fused_key_blocks(p) * p->batch * p->heads >= ((int64_t)1 << 31))
    return fail(STREAMKL_ERROR_INVALID_VALUE, std::string(what) + ": grid too large");
  (void)hipGetLastError();
  void* dqp = want_dq ? dq : nullptr;
  void* dkp = want_dk ? dk : nullptr;
  const bool causal = p->causal != 0, sk = k1 == k2;
  if (plan.path == BwdPath::kFused) {
    float* part = static_cast<float*>(workspace);
    if (setting == 1)
      dispatch_fused<1>(p->head_dim, causal, sk, s, fused_groups(p), q1, k1, q2, k2, lse1, lse2,
                        nullptr, grad_kl, dq, dk, part, stream);
    else
      dispatch_fused<2>(p->head_dim, causal, sk, s, fused_groups(p), q1, k1, q2, k2, lse1, lse2,
                        kl, grad_kl, dq, dk, part, stream);
    return check_launch(what);
  }
  if (dqp && plan.path == BwdPath::kSplitDq) {
    float* part = static_cast<float*>(workspace);
    if (setting == 1)
      dispatch_dq_split<1>(p->head_dim, causal, sk, s, plan.dq, q1, k1, q2, k2, lse1, lse2,
                           nullptr, grad_kl, dqp, part, stream);
    else
      dispatch_dq_split<2>(p->head_dim, causal, sk, s, plan.dq, q1, k1, q2, k2, lse1, lse2, kl,
                           grad_kl, dqp, part, stream);
    dqp = nullptr;
  }
  if (!dqp && !dkp) return check_launch(what);
  if (setting == 1)
    dispatch_bwd<1>(p->head_dim, causal, sk, s, q1, k1, q2, k2, lse1, lse2, nullptr, grad_kl, dqp,
                    dkp, stream);
  else
    dispatch_bwd<2>(p->head_dim, causal, sk, s, q1, k1, q2, k2, lse1, lse2, kl, grad_kl, dqp, dkp,
                    stream);
  return check_launch(what);
}

// The size bounds that validate() enforces (every size at least 1 and below 2^30, batch x heads
// below 2^30, a grid below 2^31 blocks), as a plain test. The plans are integer arithmetic on
// the sizes and are computed before validate() runs (and the size queries never run it), so
// every caller of a plan checks this first.
bool sizes_ok(const streamkl_problem_t* p) {
  if (!p || p->batch < 1 || p->heads < 1 || p->n_q < 1 || p->n_k < 1) return false;
  const int64_t lim = (int64_t)1 << 30;
  if (p->batch >= lim || p->heads >= lim || p->n_q >= lim || p->n_k >= lim ||
      p->batch * p->heads >= lim)
    return false;
  const int64_t nblk = (p->n_q > p->n_k ? p->n_q : p->n_k) / 128 + 1;
  return nblk * p->batch * p->heads < ((int64_t)1 << 31);
}

// The error of a call whose sizes fail sizes_ok(): validate()'s message.
streamkl_status_t sizes_error(const streamkl_problem_t* p, const void* q1, const void* k1,
                              const void* q2, const void* k2) {
  Shape s;
  const streamkl_status_t st = validate(p, q1, k1, q2, k2, &s);
  return st != STREAMKL_SUCCESS ? st : fail(STREAMKL_ERROR_INVALID_VALUE, "sizes out of range");
}

// The forward's adaptive choice: the split-K path when its plan cuts the keys into more than
// one range (few query blocks for the chip), else the one-pass kernel with no workspace.
size_t fwd_auto_workspace(const streamkl_problem_t* p) {
  const SplitPlan plan = split_plan(p, 0);
  return plan.nsplit > 1 ? split_workspace_bytes(p, plan.nsplit) : 0;
}

streamkl_status_t fwd_splitk_common(const streamkl_problem_t* p, const void* q1, const void* k1,
                                    const void* q2, const void* k2, float* kl, float* lse1,
                                    float* lse2, const SplitPlan& plan, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream, const char* what) {
  Shape s;
  streamkl_status_t st = validate(p, q1, k1, q2, k2, &s);
  if (st != STREAMKL_SUCCESS) return st;
  const size_t need = split_workspace_bytes(p, plan.nsplit);
  if (workspace_bytes < need)
    return fail(STREAMKL_ERROR_INVALID_VALUE,
                std::string(what) + ": workspace too small (" + std::to_string(workspace_bytes) +
                    " < " + std::to_string(need) + " bytes)");
  const int64_t n = p->batch * p->heads * p->n_q;
  const Span outs[4] = {flat_span(kl, n, 4), flat_span(lse1, n, 4), flat_span(lse2, n, 4),
                        flat_span(workspace, (int64_t)need, 1)};
  st = check_outputs(p, q1, k1, q2, k2, outs, 4, what);
  if (st != STREAMKL_SUCCESS) return st;
  if (split_blocks(s, plan) >= (1LL << 31))
    return fail(STREAMKL_ERROR_INVALID_VALUE, std::string(what) + ": grid too large");
  (void)hipGetLastError();
  const bool sk = k1 == k2, causal = p->causal != 0;
  float* part = static_cast<float*>(workspace);
#define SKL_FWDS(DD, C, S) \
  launch_fwd_split<DD, C, S>(s, plan, q1, k1, q2, k2, part, kl, lse1, lse2, stream)
  if (p->head_dim == 64) {
    if (causal) { if (sk) SKL_FWDS(64, true, true); else SKL_FWDS(64, true, false); }
    else { if (sk) SKL_FWDS(64, false, true); else SKL_FWDS(64, false, false); }
  } else {
    if (causal) { if (sk) SKL_FWDS(128, true, true); else SKL_FWDS(128, true, false); }
    else { if (sk) SKL_FWDS(128, false, true); else SKL_FWDS(128, false, false); }
  }
#undef SKL_FWDS
  return check_launch(what);
}

streamkl_status_t fwd_one_pass(const streamkl_problem_t* p, const void* q1, const void* k1,
                               const void* q2, const void* k2, float* kl, float* lse1,
                               float* lse2, hipStream_t stream, const char* what) {
  Shape s;
  streamkl_status_t st = validate(p, q1, k1, q2, k2, &s);
  if (st != STREAMKL_SUCCESS) return st;
  const int64_t n = p->batch * p->heads * p->n_q;
  const Span outs[3] = {flat_span(kl, n, 4), flat_span(lse1, n, 4), flat_span(lse2, n, 4)};
  st = check_outputs(p, q1, k1, q2, k2, outs, 3, what);
  if (st != STREAMKL_SUCCESS) return st;
  (void)hipGetLastError();
  dispatch_fwd<Bf16In>(p->head_dim, p->causal != 0, k1 == k2, s, q1, k1, q2, k2, kl, lse1, lse2,
                       1.f, 1.f, stream);
  return check_launch(what);
}

// ---------------------------------------------------------------- static scratch
// Device memory of the allocation-free forward (streamkl_fwd_noalloc): the split-K partial
// states live in this file-scope array instead of a caller workspace. Each GPU the library runs
// on holds its own copy until the process ends. In host code `scratch` names a host-side
// stand-in, not a device address: the device address of each GPU's copy is looked up once per
// device with hipGetSymbolAddress (with that device current) and only that address is used.
// The forward's default plan never needs more than 3.75 MiB of partial states: at most 256 work
// items unsplit, split into at most about 512 block items (256-row query blocks) or 1024
// wavefront items (32-row blocks), 5 floats per row and range, i.e. < 256 * 768 * 20 bytes.
constexpr size_t kScratchBytes = (size_t)4 << 20;
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

// Device address of the scratch copy on the device that `stream` belongs to (the current device
// for the null stream), where the kernels of the call run. Looked up on the first call for that
// device, with that device current (each GPU holds its own copy at its own address).
streamkl_status_t scratch_address(hipStream_t stream, void** out, const char* what) {
  int dev = -1;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess)
    return fail(STREAMKL_ERROR_HIP, std::string(what) + ": hipStreamGetDevice: " + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(STREAMKL_ERROR_NOT_SUPPORTED, std::string(what) + ": device index out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e != hipSuccess)
      return fail(STREAMKL_ERROR_HIP, std::string(what) + ": hipGetDevice: " + hipGetErrorString(e));
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(STREAMKL_ERROR_HIP, std::string(what) + ": hipSetDevice: " + hipGetErrorString(e));
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t r = hipSetDevice(cur);  // the caller's current device is left as it was
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess || !ptr)
      return fail(STREAMKL_ERROR_HIP, std::string(what) + ": hipGetSymbolAddress: " + hipGetErrorString(e));
    g_scratch_addr[dev] = ptr;
  }
  *out = g_scratch_addr[dev];
  return STREAMKL_SUCCESS;
}

}  // namespace

extern "C" {

size_t streamkl_fwd_workspace_size(const streamkl_problem_t* p) {
  if (!sizes_ok(p)) return 0;
  return fwd_auto_workspace(p);
}

streamkl_status_t streamkl_fwd(const streamkl_problem_t* p, const void* q1, const void* k1,
                               const void* q2, const void* k2, float* kl, float* lse1,
                               float* lse2, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  if (!sizes_ok(p)) return sizes_error(p, q1, k1, q2, k2);
  const SplitPlan plan = split_plan(p, 0);
  if (plan.nsplit > 1)
    return fwd_splitk_common(p, q1, k1, q2, k2, kl, lse1, lse2, plan, workspace, workspace_bytes,
                             stream, "streamkl_fwd");
  return fwd_one_pass(p, q1, k1, q2, k2, kl, lse1, lse2, stream, "streamkl_fwd");
}

streamkl_status_t streamkl_fwd_one_pass(const streamkl_problem_t* p, const void* q1,
                                        const void* k1, const void* q2, const void* k2,
                                        float* kl, float* lse1, float* lse2,
                                        hipStream_t stream) {
  return fwd_one_pass(p, q1, k1, q2, k2, kl, lse1, lse2, stream, "streamkl_fwd_one_pass");
}

size_t streamkl_fwd_noalloc_max_workspace(void) { return kScratchBytes; }

streamkl_status_t streamkl_fwd_noalloc(const streamkl_problem_t* p, const void* q1,
                                       const void* k1, const void* q2, const void* k2, float* kl,
                                       float* lse1, float* lse2, hipStream_t stream) {
  if (!sizes_ok(p)) return sizes_error(p, q1, k1, q2, k2);
  const SplitPlan plan = split_plan(p, 0);
  if (plan.nsplit <= 1)
    return fwd_one_pass(p, q1, k1, q2, k2, kl, lse1, lse2, stream, "streamkl_fwd_noalloc");
  const size_t need = split_workspace_bytes(p, plan.nsplit);
  if (need > kScratchBytes)
    return fail(STREAMKL_ERROR_NOT_SUPPORTED,
                "streamkl_fwd_noalloc: the split-K partial states need " + std::to_string(need) +
                    " bytes, more than the " + std::to_string(kScratchBytes) +
                    " bytes of the library's scratch; use streamkl_fwd with a workspace");
  // validation first (inputs, outputs, overlaps): an invalid call makes no device call at all,
  // not even the scratch lookup
  Shape s;
  streamkl_status_t st = validate(p, q1, k1, q2, k2, &s);
  if (st != STREAMKL_SUCCESS) return st;
  const int64_t n = p->batch * p->heads * p->n_q;
  const Span outs[3] = {flat_span(kl, n, 4), flat_span(lse1, n, 4), flat_span(lse2, n, 4)};
  st = check_outputs(p, q1, k1, q2, k2, outs, 3, "streamkl_fwd_noalloc");
  if (st != STREAMKL_SUCCESS) return st;
  void* ws = nullptr;
  st = scratch_address(stream, &ws, "streamkl_fwd_noalloc");
  if (st != STREAMKL_SUCCESS) return st;
  return fwd_splitk_common(p, q1, k1, q2, k2, kl, lse1, lse2, plan, ws, kScratchBytes, stream,
                           "streamkl_fwd_noalloc");
}

streamkl_status_t streamkl_fwd_fp8(const streamkl_problem_t* p, float descale1, float descale2,
                                   const void* q1, const void* k1, const void* q2, const void* k2,
                                   float* kl, float* lse1, float* lse2, hipStream_t stream) {
  Shape s;
  streamkl_status_t st = validate(p, q1, k1, q2, k2, &s, 1);
  if (st != STREAMKL_SUCCESS) return st;
  if (!(descale1 > 0.f) || !(descale1 < __builtin_huge_valf()) || !(descale2 > 0.f) ||
      !(descale2 < __builtin_huge_valf()))
    return fail(STREAMKL_ERROR_INVALID_VALUE, "streamkl_fwd_fp8: descales must be finite and > 0");
  const int64_t n = p->batch * p->heads * p->n_q;
  const Span outs[3] = {flat_span(kl, n, 4), flat_span(lse1, n, 4), flat_span(lse2, n, 4)};
  st = check_outputs(p, q1, k1, q2, k2, outs, 3, "streamkl_fwd_fp8", 1);
  if (st != STREAMKL_SUCCESS) return st;
  (void)hipGetLastError();
  dispatch_fwd<Fp8In>(p->head_dim, p->causal != 0, k1 == k2, s, q1, k1,
                      q2, k2, kl, lse1, lse2, descale1, descale2, stream);
  return check_launch("streamkl_fwd_fp8");
}

int32_t streamkl_fwd_splitk_default_splits(const streamkl_problem_t* p) {
  if (!sizes_ok(p)) return 0;
  return split_plan(p, 0).nsplit;
}

size_t streamkl_fwd_splitk_workspace_size(const streamkl_problem_t* p, int32_t n_splits) {
  if (!sizes_ok(p)) return 0;
  return split_workspace_bytes(p, split_plan(p, n_splits).nsplit);
}

streamkl_status_t streamkl_fwd_splitk(const streamkl_problem_t* p, const void* q1,
                                      const void* k1, const void* q2, const void* k2, float* kl,
                                      float* lse1, float* lse2, int32_t n_splits,
                                      void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
  if (!sizes_ok(p)) return sizes_error(p, q1, k1, q2, k2);
  return fwd_splitk_common(p, q1, k1, q2, k2, kl, lse1, lse2, split_plan(p, n_splits), workspace,
                           workspace_bytes, stream, "streamkl_fwd_splitk");
}

size_t streamkl_bwd_workspace_size(const streamkl_problem_t* p) {
  if (!sizes_ok(p) || (p->head_dim != 64 && p->head_dim != 128)) return 0;
  return bwd_auto_plan(p).workspace;
}

streamkl_status_t streamkl_bwd_fixP1(const streamkl_problem_t* p, const void* q1,
                                     const void* k1, const void* q2, const void* k2,
                                     const float* lse1, const float* lse2, const float* grad_kl,
                                     void* dq2, void* dk2, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  return bwd_common(p, 1, q1, k1, q2, k2, lse1, lse2, nullptr, grad_kl, dq2, dk2, true, true,
                    stream, "streamkl_bwd_fixP1", BwdMode::kAuto, 0, workspace, workspace_bytes);
}

streamkl_status_t streamkl_bwd_fixP2(const streamkl_problem_t* p, const void* q1,
                                     const void* k1, const void* q2, const void* k2,
                                     const float* lse1, const float* lse2, const float* kl,
                                     const float* grad_kl, void* dq1, void* dk1, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  return bwd_common(p, 2, q1, k1, q2, k2, lse1, lse2, kl, grad_kl, dq1, dk1, true, true, stream,
                    "streamkl_bwd_fixP2", BwdMode::kAuto, 0, workspace, workspace_bytes);
}

streamkl_status_t streamkl_bwd_dq(const streamkl_problem_t* p, int32_t setting, const void* q1,
                                  const void* k1, const void* q2, const void* k2,
                                  const float* lse1, const float* lse2, const float* kl,
                                  const float* grad_kl, void* dq, hipStream_t stream) {
  return bwd_common(p, setting, q1, k1, q2, k2, lse1, lse2, kl, grad_kl, dq, nullptr, true, false,
                    stream, "streamkl_bwd_dq", BwdMode::kOneKernel);
}

streamkl_status_t streamkl_bwd_dk(const streamkl_problem_t* p, int32_t setting, const void* q1,
                                  const void* k1, const void* q2, const void* k2,
                                  const float* lse1, const float* lse2, const float* kl,
                                  const float* grad_kl, void* dk, hipStream_t stream) {
  return bwd_common(p, setting, q1, k1, q2, k2, lse1, lse2, kl, grad_kl, nullptr, dk, false, true,
                    stream, "streamkl_bwd_dk", BwdMode::kOneKernel);
}

int32_t streamkl_bwd_dq_splitk_default_splits(const streamkl_problem_t* p) {
  if (!sizes_ok(p)) return 0;
  return dq_split_plan(p, 0).nsplit;
}

size_t streamkl_bwd_dq_splitk_workspace_size(const streamkl_problem_t* p, int32_t n_splits) {
  if (!sizes_ok(p)) return 0;
  return dq_split_workspace_bytes(p, dq_split_plan(p, n_splits).nsplit);
}

streamkl_status_t streamkl_bwd_dq_splitk(const streamkl_problem_t* p, int32_t setting,
                                         const void* q1, const void* k1, const void* q2,
                                         const void* k2, const float* lse1, const float* lse2,
                                         const float* kl, const float* grad_kl, void* dq,
                                         int32_t n_splits, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream) {
  return bwd_common(p, setting, q1, k1, q2, k2, lse1, lse2, kl, grad_kl, dq, nullptr, true, false,
                    stream, "streamkl_bwd_dq_splitk", BwdMode::kSplitDq, n_splits, workspace,
                    workspace_bytes);
}

size_t streamkl_bwd_fused_workspace_size(const streamkl_problem_t* p) {
  if (!sizes_ok(p) || p->n_q > kFusedMaxQ || (p->head_dim != 64 && p->head_dim != 128))
    return 0;
  return fused_workspace_bytes(p);
}

streamkl_status_t streamkl_bwd_fused(const streamkl_problem_t* p, int32_t setting, const void* q1,
                                     const void* k1, const void* q2, const void* k2,
                                     const float* lse1, const float* lse2, const float* kl,
                                     const float* grad_kl, void* dq, void* dk, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  return bwd_common(p, setting, q1, k1, q2, k2, lse1, lse2, kl, grad_kl, dq, dk, true, true,
                    stream, "streamkl_bwd_fused", BwdMode::kFused, 0, workspace,
                    workspace_bytes);
}

const char* streamkl_status_string(streamkl_status_t status) {
  // a C caller may pass any int: read the bytes, since loading an out-of-range value as the
  // enum type is undefined in C++
  int code;
  static_assert(sizeof(code) == sizeof(status), "the status enum is int-sized");
  std::memcpy(&code, &status, sizeof(code));
  switch (code) {
    case STREAMKL_SUCCESS: return "STREAMKL_SUCCESS";
    case STREAMKL_ERROR_INVALID_VALUE: return "STREAMKL_ERROR_INVALID_VALUE";
    case STREAMKL_ERROR_NOT_SUPPORTED: return "STREAMKL_ERROR_NOT_SUPPORTED";
    case STREAMKL_ERROR_HIP: return "STREAMKL_ERROR_HIP";
    default: return "STREAMKL_UNKNOWN_STATUS";
  }
}

const char* streamkl_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
