// bf16 MFMA GEMM for gfx950: C[M][N] = A[M][K] B[N][K]^T (+ Ae Be^T), fp32 accumulate.
//
// This is the dense contraction of every base projection of the QLoRA layer
// (the pages' profiling remark: runtime is dominated by the large MLP
// matmuls; Show HN thread) with the rank-r LoRA product folded in as a
// K-extension: for Y = X W^T + s (X A^T) B^T the caller passes
// Ae = [hi(sU) | lo(sU)] and Be = [B | B] (U = X A^T formed first, so the
// merged weight W + s B A never exists; Mistral benchmark page, items 10-11).
// hi/lo is a two-term bf16 split of the fp32 product, which keeps the LoRA
// term accurate to ~2^-17 relative on bf16 matrix cores.
//
// gemm_bf16_kernel: 256 x 256 output tile per workgroup of 4 waves (one per
// SIMD) laid out 2 x 2, each wave 128 x 128 = 4 x 4 MFMA 32x32x16 tiles (256
// fp32 accumulators per lane). K is walked in 64-wide steps. Operands reach
// LDS through buffer loads straight into LDS (one buffer resource per operand
// tile, so rows past M or N read as zeros), into a ring of five 32 KB
// half-stage slots (one operand of one step each): while a step reads two
// slots, the next step and a half are in flight. The 1 KB load blocks are
// unpadded and XOR-swizzled so that the ds_read_b128 fragment reads stay
// conflict-free; the MFMA row order is permuted to match and undone in the
// epilogue. Fragments of the next substep are read while the matrix cores
// work on the current one, and sched_group_barrier hints interleave the LDS
// reads and load issues with the MFMAs. With a bf16 B operand the last
// k-step also loads what the tile needs after its main loop (the
// K-extension's first step into free ring slots, the row-product operands,
// the first g/u slab of the ACT_BWD epilogue), and the K-extension's later
// steps load while the previous one multiplies.
// Optional extras: A split along K into up to three matrices (dX = sum of
// dY_p W_p over separately stored dY_p), and an epilogue that writes column
// ranges to three outputs (q, k, v from one GEMM).
//
// B operand: bf16 rows (a staged dequant, or 16-bit base weights), or NF4
// codes dequantized into the ring by the workgroup itself (BSRC_NF4,
// BSRC_NF4_PAIR, BSRC_NF4_T): 4-bit codes and an absmax per 64 weights
// (8 KB + 1 KB per step instead of 32 KB of bf16) come into registers a step
// ahead, and each thread forms bf16_rne(fp32_rne(level[code] * absmax)) for
// its 64 weights with byte permutes from a per-step table, exactly as the
// standalone dequant. The order of every instruction of such a step is fixed
// in the source, so that the dequant work sits between the MFMAs. BSRC_NF4_T
// reads the weight transposed (the backward dX = dY W): its slot is k-major,
// and the B fragments come from LDS transpose reads.
//
// Epilogues: each wave stages a 32-row slab of its
// accumulators through its own LDS region, so only wave-local ordering is
// needed, reads a slab's staged values back in one batch (one LDS wait per
// slab) and stores 16 bytes per lane. The gated epilogues take the
// activation as a compile-time constant (one branch per launch, none per
// value): with one wave per SIMD the epilogue runs with the matrix cores
// idle, so its instruction count matters.
//
// Row products (gemm_bf16_kernel, GATEUP and ACT_BWD, on request): the bf16
// values the epilogue writes (H; dg and du) are also multiplied by a rank-r
// operand (A_down; blockdiag(B_gate, B_up)) on MFMA 16x16x32, from a panel
// that overwrites each staged row once it is read. The results are parked
// in LDS per slab; after the last slab the two waves of a tile row add their
// column halves and store one fp32 partial per tile column. The MLP's next
// LoRA product then needs no pass that reads H or dg|du back.
//
// Split-K (gemm_bf16_kernel, store epilogues only): an output with fewer than
// 256 tiles is computed as several K ranges that write fp32 partials;
// splitk_reduce_kernel sums them in a fixed order and stores bf16.
//
// Tile order: workgroup ids are dealt to the 8 XCDs round-robin; ids are
// remapped so that each XCD walks a contiguous range of tiles, grouped 8
// M-tiles at a time, which keeps shared A rows / B columns in that XCD's L2.
#include "common.hpp"
#include "kernels.hpp"
#include "nf4_table.hpp"

#include <type_traits>

namespace qlora {

namespace {

constexpr int BM = 256, BN = 256, BK = 64;

__device__ __forceinline__ int xcd_remap(int pid, int n) {
  const int X = 8;
  int q = n / X, rmd = n % X;
  int xcd = pid % X, local = pid / X;
  return (xcd < rmd ? xcd * (q + 1) : rmd * (q + 1) + (xcd - rmd) * q) + local;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// LDS store the compiler does not track: it is not ordered against the DMA
// still in flight to other LDS regions (the compiler would otherwise wait for
// all of them). Completion is covered by the lgkmcnt(0) of wait_vm<>.
__device__ __forceinline__ void lds_store16(void* p, u32x4_t v) {
  const uint32_t off = (uint32_t)(uintptr_t)(lds_ptr_t)p;
  asm volatile("ds_write_b128 %0, %1" : : "v"(off), "v"(v) : "memory");
}

// Wait until at most N vector-memory loads of this wave are outstanding and
// all of its LDS operations are done (expcnt left unconstrained).
// gfx9 encoding: vmcnt[3:0] | vmcnt[5:4] << 14, expcnt[6:4], lgkmcnt[11:8].
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

// Workgroup barrier without the memory fence of __syncthreads(): the fence
// would wait for every DMA in flight (vmcnt(0)). Waves wait for their own
// DMA with wait_vm<> first, so after the barrier every wave's data for that
// stage is in LDS. The empty asm keeps the compiler from moving LDS accesses
// across the barrier.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Orders one wave's LDS accesses across its lanes (a lane reads what another
// lane of the same wave wrote). LDS serves a wave's instructions in issue
// order, so only the compiler has to be held back. Unlike __syncthreads() it
// waits for nothing: the global stores in flight keep going.
__device__ __forceinline__ void wave_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

// This lane's index in the wave, computed where it is used. Being volatile,
// it is neither merged with an earlier copy nor kept live across the code
// before it: a value the register allocator spilled would be reloaded from
// scratch, and that load's wait would also wait for every store issued
// before it.
__device__ __forceinline__ int lane_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

}  // namespace

constexpr uint32_t kNf4Lev[16] = {QLORA_NF4_LEVEL_BITS};

// ===========================================================================
// bf16-B GEMM: one 256 x 256 tile per workgroup of 4 waves (1 per SIMD), each
// wave 128 x 128 = 4 x 4 MFMA 32x32x16 tiles, its 256 fp32 accumulators in
// AGPRs. This is the kernel of the staged path (B = pre-dequantized weight).
//
// Operand feed: buffer loads straight into LDS (buffer_load_dwordx4 ... lds),
// through a buffer resource per tile whose size ends at the matrix end, so
// rows past M (N) read as zeros without per-row clamps. One load instruction
// fills a 1 KB block with 8 rows x 128 B (full 128-byte lines). Blocks are
// unpadded; inside each 256-byte unit of block q, 16-byte position p holds
// logical position p ^ (q & 15). The MFMA lanes read rows in the order below,
// so the 16 lanes of a ds_read_b128 phase read 16 consecutive blocks and hit
// 16 different bank groups:
//   MFMA row i (0..31) of tile t of wave w reads tile row
//   8 * (16 * w + (i & 15)) + 2 * t + (i >> 4)          (A; B likewise).
// The epilogue undoes this permutation.
//
// Pipeline per 64-wide k-step: a ring of five half-stage slots (A or B of one
// step each). Step s reads two slots; over its first three substeps it issues
// B of step s+1 and A of step s+2 into the two slots freed by step s-1, then
// waits for step s+1's halves only; one barrier per step.
// ===========================================================================
namespace {
constexpr int G_SLOT = 32768;           // one operand (256 rows x 64 bf16) of one k-step

// buffer load of `size` bytes per lane into LDS at lds + size*lane; the
// resource is rebuilt from uniform integers at each use (it stays in SGPRs)
template <int SIZE>
__device__ __forceinline__ void bload_lds(uint64_t base, int nrec, void* lds, uint32_t voff, int soff) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(((uint64_t)hi << 32) | lo), (short)0, __builtin_amdgcn_readfirstlane(nrec), 0x00020000);
  const int so = __builtin_amdgcn_readfirstlane(soff);
  if constexpr (SIZE == 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, so, 0, 0);
  else __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 4, voff, so, 0, 0);
}

// bytes a buffer resource covers for `rows` rows of pitch `ld` bf16, capped
// at the 31-bit record limit (integer arithmetic throughout)
__device__ __forceinline__ int rec_bytes(int64_t rows, int64_t ld) {
  const int64_t b = rows * ld * 2;
  return b < 0x7fffffff ? (int)b : 0x7fffffff;
}

// offset that no buffer covers: the load returns zeros
constexpr uint32_t OOB = 0x80000000u;

// buffer resource over nrec bytes at base (uniform values, kept in SGPRs)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(uint64_t base, int nrec) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0,
                                           __builtin_amdgcn_readfirstlane(nrec), 0x00020000);
}

// Wait until at most N vector-memory loads of this wave are outstanding; LDS
// operations are not waited for.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
}  // namespace

template <int EPI, bool SEGA, int BSRC>
__global__ __launch_bounds__(256)
void gemm_bf16_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[5 * G_SLOT];   // all 160 KB of LDS
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  const int ntm = (p.M + BM - 1) / BM, ntn = (p.N + BN - 1) / BN;
  // job -> (tile, K split); the splits of a tile are consecutive job ids
  const int nsplit = p.splits > 1 ? p.splits : 1;
  const int job = xcd_remap(blockIdx.x, ntm * ntn * nsplit);
  const int ksp = job % nsplit;
  const int pid = job / nsplit;
  const int GM = 8;
  const int per_group = GM * ntn;
  const int group = pid / per_group;
  const int first_m = group * GM;
  const int gsz = min(ntm - first_m, GM);
  const int tm = first_m + (pid % per_group) % gsz;
  const int tn = (pid % per_group) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;
  // every row and column of the tile is inside the output: the epilogue then
  // runs without per-row bounds checks (no predicated stores, no merged
  // zero/value registers)
  const bool interior = m0 + BM <= p.M && n0 + BN <= p.N;
  const int nk = p.K / BK;
  // this job's k-steps [kt0, kt1) (the host keeps every split non-empty)
  const int kper = (nk + nsplit - 1) / nsplit;
  const int kt0 = ksp * kper, kt1 = min(nk, kt0 + kper);

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // ---- operand ring ----
  // Five 32 KB slots. Half-stage H_i, counted from this job's first k-step
  // (H_2s = the A operand of step kt0 + s, H_2s+1 = its B operand), lives in
  // slot i % 5: while a step reads two slots, the other three hold the next
  // one and a half steps. A slot is 32 DMA blocks of 1 KB; block q holds tile
  // rows 8q..8q+7 (64 bf16 each) at byte 1024 q. In each 256-byte unit u of a
  // block (rows 2u, 2u+1), 16-byte position p holds logical position
  // p ^ (q & 15), logical = (row & 1) * 8 + chunk. The 16 lanes of a fragment
  // read take one logical position from 16 consecutive blocks, so they hit 16
  // different bank groups without padding; the ring then fits LDS.
  const int64_t rowsA = min(BM, p.M - m0), rowsB = min(BN, p.N - n0);
  const uint64_t bA = (uint64_t)(p.A + (int64_t)m0 * p.lda), bB = (uint64_t)(p.B + (int64_t)n0 * p.ldb);
  const int nA = rec_bytes(rowsA, p.lda);
  const int nB = rec_bytes(rowsB, p.ldb);

  // ---- NF4 B operand (BSRC other than BSRC_BF16) ----
  // The B half-stage of a step is written, not loaded: each thread turns the
  // 64 codes of one weight row and one 64-wide block (one absmax; brought
  // into registers a step ahead) into bf16 and stores them in LDS. Values are
  // bf16_rne(fp32_rne(level * absmax)), the contract of the dequant kernels:
  // the 16 possible values of the thread's block are formed once per step
  // (that product and rounding, for each level) and each code selects one
  // with byte permutes.
  //   Row-major (NF4, NF4_PAIR): a thread owns one tile row R (the weight row
  //     of output column n0 + R, 64 codes of the step); its stores fill the
  //     slot layout above, chunk (j + f) & 7 in store j with f = 2 ((lane >> 1)
  //     & 3) so that the 16 lanes of each store phase hit 16 different
  //     positions. Waves 0, 1 own gate rows, waves 2, 3 up rows (in pair mode
  //     they read different weights).
  //   Transposed (NF4_T): the tile's K rows are weight rows, its columns the
  //     weight's features. Lane l owns weight row l of the step, wave w
  //     features 64 w .. 64 w + 63 of the tile. The slot is k-major: row k
  //     (512 bytes) holds feature n = 8 x + y at position p = 32 y + x, and
  //     16-byte chunk c of the row at physical chunk c ^ sw(k). A thread's
  //     store y writes its 8 features 8 x + y (x = 8 w .. 8 w + 7). The B
  //     fragments are read with the LDS transpose read (ds_read_b64_tr_b16),
  //     which gives each lane of a 16-lane group 4 consecutive K values of
  //     its own column; the swizzle keeps both the stores and these reads
  //     free of bank conflicts.
  constexpr bool NF4 = BSRC != BSRC_BF16;
  constexpr bool NT = BSRC == BSRC_NF4_T;
  constexpr int NQ = NT ? 3 : 5;      // loads per thread per step
  constexpr int NPART = 56;           // dequant parts per step
  constexpr int NPRE = 8;             // of them done in the fourth substep of the step before
  static_assert(NPART - NPRE == 48, "one dequant part per MFMA of substeps 0-2");
  struct QRegs {
    uint32_t c[8];
    float a[1];
  };
  uint64_t qcb0 = 0, qsb0 = 0, qcb1 = 0, qsb1 = 0;   // codes / absmax bases (NF4_T: weights 0, 1)
  int qcn0 = 0, qsn0 = 0, qcn1 = 0, qsn1 = 0;        // their buffer sizes in bytes
  uint32_t qvo[4] = {0u, 0u, 0u, 0u}, qso = 0u;      // per-lane byte offsets of the loads
  uint32_t woff[8];                                 // byte offsets of the 8 stores in a slot
  uint32_t tboff[2][4];                             // NF4_T: B fragment read offsets [half][tile]
  int kq1 = nk;                                     // NF4_T: first k-step of weight 1
  const int qk2 = p.K / 2, qn2 = p.N / 2;
  auto tsw = [](int k) { return 2 * (k & 1) + 8 * ((k >> 1) & 1) + ((k >> 2) & 1) + 4 * ((k >> 3) & 1); };
  if constexpr (NF4) {
    if constexpr (!NT) {
      const int R = 128 * (wave & 1) + 64 * (lane >> 5) + 32 * (wave >> 1) + (lane & 31);
      const int gn = n0 + R;
      int64_t wrow = gn, wrows = p.N;
      const uint8_t* codes = p.codes0;
      const float* am = p.absmax0;
      if (BSRC == BSRC_NF4_PAIR) {
        wrow = (int64_t)(gn >> 6) * 32 + (gn & 31);
        wrows = p.N / 2;
        if (wave >= 2) { codes = p.codes1; am = p.absmax1; }
      }
      // rows at or past the weight's end read as zeros: level 0 times absmax 0
      qcb0 = (uint64_t)codes;
      qcn0 = (int)min<int64_t>(wrows * qk2, 0x7fffffff);
      qsb0 = (uint64_t)am;
      qsn0 = (int)min<int64_t>(wrows * (p.K / 64) * 4, 0x7fffffff);
      const bool in = wrow < wrows;
      const int f = 2 * ((lane >> 1) & 3);
#pragma unroll
      for (int i = 0; i < 4; ++i) qvo[i] = in ? (uint32_t)(wrow * qk2) + (uint32_t)(((f + 2 * i) & 7) * 4) : OOB;
      qso = in ? (uint32_t)(wrow * (p.K / 64) * 4) : OOB;
      const int q = R >> 3, u = (R & 7) >> 1;
#pragma unroll
      for (int j = 0; j < 8; ++j) woff[j] = q * 1024 + u * 256 + ((((R & 1) * 8 + ((j + f) & 7)) ^ (q & 15)) * 16);
    } else {
      const int64_t rows0 = p.ksplit > 0 ? p.ksplit : p.K;
      kq1 = p.ksplit > 0 ? p.ksplit / BK : nk;
      qcb0 = (uint64_t)p.codes0;
      qcn0 = (int)min<int64_t>(rows0 * qn2, 0x7fffffff);
      qsb0 = (uint64_t)p.absmax0;
      qsn0 = (int)min<int64_t>(rows0 * (p.N / 64) * 4, 0x7fffffff);
      if (p.ksplit > 0) {
        qcb1 = (uint64_t)p.codes1;
        qcn1 = (int)min<int64_t>((p.K - rows0) * qn2, 0x7fffffff);
        qsb1 = (uint64_t)p.absmax1;
        qsn1 = (int)min<int64_t>((p.K - rows0) * (p.N / 64) * 4, 0x7fffffff);
      }
      // features at or past N (a whole wave's block, N being a multiple of
      // 64) read as zeros
      const int f0 = n0 + 64 * wave;
      const bool in = f0 < p.N;
      qvo[0] = in ? (uint32_t)lane * (uint32_t)qn2 + (uint32_t)(f0 / 2) : OOB;
      qvo[1] = qvo[0] + (in ? 16u : 0u);
      qso = in ? ((uint32_t)lane * (uint32_t)(p.N / 64) + (uint32_t)(f0 / 64)) * 4u : OOB;
#pragma unroll
      for (int y = 0; y < 8; ++y) woff[y] = lane * 512 + (((4 * y + wave) ^ tsw(lane)) << 4);
      // fragment reads: lane L of a 16-lane group g supplies, for the group's
      // element e = (L & 15) >> 2, the 4 columns starting at 16 wn + 4 (L & 3)
      // of feature class y = 2 nt + (g & 1), K row 8 (L >> 5) + 4 half + e
      const int e = (lane & 15) >> 2, a4 = lane & 3;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const int k = 8 * (lane >> 5) + 4 * h + e;
          const int pos = (2 * nt + ((lane >> 4) & 1)) * 32 + 16 * wn + 4 * a4;
          tboff[h][nt] = k * 512 + ((((pos >> 3) ^ tsw(k)) << 4) | ((pos & 7) << 1));
        }
    }
  }
  // codes and absmax of k-step kt into r
  auto issue_q = [&](int kt, QRegs& r) {
    if constexpr (!NT) {
      const __amdgpu_buffer_rsrc_t rc = make_rsrc(qcb0, qcn0), rs = make_rsrc(qsb0, qsn0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(rc, qvo[i], kt * 32, 0);
        r.c[2 * i] = v[0];
        r.c[2 * i + 1] = v[1];
      }
      r.a[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, qso, kt * 4, 0));
    } else {
      const bool w1 = kt >= kq1;
      const int kl = w1 ? kt - kq1 : kt;
      const __amdgpu_buffer_rsrc_t rc = make_rsrc(w1 ? qcb1 : qcb0, w1 ? qcn1 : qcn0);
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(w1 ? qsb1 : qsb0, w1 ? qsn1 : qsn0);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rc, qvo[i], kl * BK * qn2, 0);
#pragma unroll
        for (int t = 0; t < 4; ++t) r.c[4 * i + t] = v[t];
      }
      r.a[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, qso, kl * BK * (p.N / 64) * 4, 0));
    }
  };
  // byte b of the result: plane byte s_b of value (s_b + 8 * bit 3) where the
  // selector bytes s hold the low 3 bits and m holds b + 4 * bit 3. P[0..3]
  // hold the low bytes of the 16 values (4 per register), P[4..7] the high.
  auto qlook = [](const uint32_t* P, uint32_t sel, uint32_t m) {
    return __builtin_amdgcn_perm(__builtin_amdgcn_perm(P[3], P[2], sel), __builtin_amdgcn_perm(P[1], P[0], sel), m);
  };
  // The table in parts: parts 0-3 form two of its bf16 pairs each, parts 4-5
  // two plane registers each.
  auto qtable_part = [&](int part, const QRegs& r, uint32_t (&D)[8], uint32_t (&P)[8]) {
    if (part < 4) {
#pragma unroll
      for (int i = 2 * part; i < 2 * part + 2; ++i)
        D[i] = pack_bf16x2(__builtin_bit_cast(float, kNf4Lev[2 * i]) * r.a[0],
                           __builtin_bit_cast(float, kNf4Lev[2 * i + 1]) * r.a[0]);
    } else {
#pragma unroll
      for (int k = 2 * (part - 4); k < 2 * (part - 4) + 2; ++k) {
        P[k] = __builtin_amdgcn_perm(D[2 * k + 1], D[2 * k], 0x06040200u);
        P[4 + k] = __builtin_amdgcn_perm(D[2 * k + 1], D[2 * k], 0x07050301u);
      }
    }
  };
  // A step's dequant in NPART parts of about 4 VALU instructions each, which
  // the main loop places one per MFMA. Code dword c holds elements 8 c ..
  // 8 c + 7 of the thread's block (element 2 m in the high nibble of byte m).
  // Per dword: part 0 the lookup selectors, 1 the merge selectors, 2 the
  // low-byte lookups, 3 the high-byte lookups; row-major then 4-5 the
  // interleave into bf16 pairs and 6 the store (chunk = dword); transposed 4
  // the pairs (element y, element y + 2) of the dword, then (per two dwords
  // 2 q, 2 q + 1) two parts forming word q of the 8 stores, and after all
  // dwords the 8 stores (store y: elements 8 x + y).
  struct QStep {
    uint32_t s0[8], s1[8], m0[8], m1[8], a0[8], a1[8], b0[8], b1[8];
    uint32_t ev[8][4];
    u32x4_t o[8];
  };
  auto qpart = [&](QStep& S, int pp, const QRegs& r, const uint32_t (&P)[8], uint8_t* sbase) {
    // decode part pp into (kind, dword c / store y / pair q)
    int kind, c = 0;
    if constexpr (!NT) {
      c = pp / 7;
      kind = pp % 7;
    } else if (pp < 48) {
      const int q = pp / 12, rr = pp % 12;
      if (rr < 10) { c = 2 * q + rr / 5; kind = rr % 5; }
      else { c = q; kind = 8 + (rr - 10); }   // pair q, half 0 / 1
    } else {
      c = pp - 48;
      kind = 10;                               // store y = c
    }
    if (kind == 0) {
      const uint32_t d = r.c[c];
      S.s0[c] = d & 0x07070707u;                          // low nibbles: elements 1, 3, 5, 7
      S.s1[c] = (d >> 4) & 0x07070707u;                   // high nibbles: elements 0, 2, 4, 6
    } else if (kind == 1) {
      const uint32_t d = r.c[c];
      S.m0[c] = ((d >> 1) & 0x04040404u) | 0x03020100u;
      S.m1[c] = ((d >> 5) & 0x04040404u) | 0x03020100u;
    } else if (kind == 2) {
      S.a0[c] = qlook(P, S.s0[c], S.m0[c]);
      S.a1[c] = qlook(P, S.s1[c], S.m1[c]);
    } else if (kind == 3) {
      S.b0[c] = qlook(P + 4, S.s0[c], S.m0[c]);
      S.b1[c] = qlook(P + 4, S.s1[c], S.m1[c]);
    } else if (!NT && kind == 4) {
      S.ev[c][0] = __builtin_amdgcn_perm(S.a0[c], S.a1[c], 0x05010400u);
      S.ev[c][1] = __builtin_amdgcn_perm(S.b0[c], S.b1[c], 0x05010400u);
      S.ev[c][2] = __builtin_amdgcn_perm(S.a0[c], S.a1[c], 0x07030602u);
      S.ev[c][3] = __builtin_amdgcn_perm(S.b0[c], S.b1[c], 0x07030602u);
    } else if (!NT && kind == 5) {
      S.o[c][0] = __builtin_amdgcn_perm(S.ev[c][1], S.ev[c][0], 0x05010400u);
      S.o[c][1] = __builtin_amdgcn_perm(S.ev[c][1], S.ev[c][0], 0x07030602u);
      S.o[c][2] = __builtin_amdgcn_perm(S.ev[c][3], S.ev[c][2], 0x05010400u);
      S.o[c][3] = __builtin_amdgcn_perm(S.ev[c][3], S.ev[c][2], 0x07030602u);
    } else if (!NT && kind == 6) {
      lds_store16(sbase + woff[c], S.o[c]);
    } else if (NT && kind == 4) {
      // bf16 pairs of one dword: elements (0, 2), (4, 6), (1, 3), (5, 7)
      S.ev[c][0] = __builtin_amdgcn_perm(S.b1[c], S.a1[c], 0x05010400u);
      S.ev[c][1] = __builtin_amdgcn_perm(S.b1[c], S.a1[c], 0x07030602u);
      S.ev[c][2] = __builtin_amdgcn_perm(S.b0[c], S.a0[c], 0x05010400u);
      S.ev[c][3] = __builtin_amdgcn_perm(S.b0[c], S.a0[c], 0x07030602u);
    } else if (NT && kind < 10) {
      // dwords 2 q, 2 q + 1 -> word q of stores y (half 0: y = 0..3, 1: 4..7):
      // (element y of 2 q, element y of 2 q + 1)
      const int q = c;
#pragma unroll
      for (int y = 4 * (kind - 8); y < 4 * (kind - 8) + 4; ++y) {
        const int src = (y & 1) ? 2 + ((y >> 2) & 1) : ((y >> 2) & 1);   // ev index
        const uint32_t sel = ((y >> 1) & 1) ? 0x07060302u : 0x05040100u;
        S.o[y][q] = __builtin_amdgcn_perm(S.ev[2 * q + 1][src], S.ev[2 * q][src], sel);
      }
    } else if (NT) {
      lds_store16(sbase + woff[c], S.o[c]);
    }
  };
  // DMA: wave w, load j (0..7) fills block q = 8w + j; lane l writes position
  // l of it. Tile row and first column of that position:
  auto drow = [&](int j) {
    const int pl = (lane & 15) ^ ((8 * wave + j) & 15);
    return 8 * (8 * wave + j) + 2 * (lane >> 4) + (pl >> 3);
  };
  auto dcol = [&](int j) { return (((lane & 15) ^ ((8 * wave + j) & 15)) & 7) * 8; };
  // A operand of k-step kt. SEGA: K is split into up to three segments, each
  // its own matrix with its own row pitch (segment starts are multiples of
  // BK, so a step never straddles two). The per-lane offsets are formed from
  // the segment's pitch at each use (sk: the segment's first byte along K).
  // Plain scalars, not a struct, so that everything stays in SGPRs.
  uint64_t sb0 = 0, sb1 = 0, sb2 = 0;
  int sn0 = 0, sn1 = 0, sn2 = 0, sk1 = 0, sk2 = 0;
  uint32_t sl0 = 0, sl1 = 0, sl2 = 0;
  int ks1 = nk, ks2 = nk;
  if constexpr (SEGA) {
    ks1 = p.ka1 / BK;
    ks2 = p.ka2 / BK;
    sb0 = bA; sn0 = nA; sl0 = (uint32_t)(p.lda * 2);
    sb1 = (uint64_t)(p.A1 + (int64_t)m0 * p.lda1);
    sn1 = rec_bytes(rowsA, p.lda1);
    sl1 = (uint32_t)(p.lda1 * 2);
    sk1 = ks1 * BK * 2;
    sb2 = (uint64_t)(p.A2 + (int64_t)m0 * p.lda2);
    sn2 = rec_bytes(rowsA, p.lda2);
    sl2 = (uint32_t)(p.lda2 * 2);
    sk2 = ks2 * BK * 2;
  }
  // (base, records, pitch, first K byte) of step kt's segment, as sums of
  // 0/1 flags times differences (a select chain here was lowered to an
  // indexed stack array)
  auto aseg = [&](int kt, uint64_t& b, int& n, uint32_t& l, int& k) {
    const int f1 = kt >= ks1, f2 = kt >= ks2;
    b = sb0 + (uint64_t)f1 * (sb1 - sb0) + (uint64_t)f2 * (sb2 - sb1);
    n = sn0 + f1 * (sn1 - sn0) + f2 * (sn2 - sn1);
    l = sl0 + (uint32_t)f1 * (sl1 - sl0) + (uint32_t)f2 * (sl2 - sl1);
    k = f1 * sk1 + f2 * (sk2 - sk1);
  };
  auto slot = [&](int i) { return smem + (i % 5) * G_SLOT; };
  auto issue_half = [&](int i, int j) {   // this wave's load j of half-stage H_i
    const int kt = kt0 + (i >> 1), kb = kt * BK * 2;
    uint8_t* dst = slot(i) + (8 * wave + j) * 1024;
    if ((i & 1) == 0) {
      if constexpr (SEGA) {
        uint64_t b; int n; uint32_t l; int k;
        aseg(kt, b, n, l, k);
        bload_lds<16>(b, n, dst, (uint32_t)drow(j) * l + (uint32_t)dcol(j) * 2u, kb - k);
      } else {
        bload_lds<16>(bA, nA, dst, (uint32_t)(drow(j) * p.lda + dcol(j)) * 2u, kb);
      }
    } else {
      bload_lds<16>(bB, nB, dst, (uint32_t)(drow(j) * p.ldb + dcol(j)) * 2u, kb);
    }
  };

  // ---- fragments ----
  // tile mt of substep ks: block 16*wm + (lane & 15), unit mt, logical position
  // ((lane >> 4) & 1) * 8 + 2 ks + (lane >> 5)
  const int fq = (16 * wm + (lane & 15)) * 1024, gq = (16 * wn + (lane & 15)) * 1024;
  auto fpos = [&](int ks) { return ((((lane >> 4) & 1) * 8 + 2 * ks + (lane >> 5)) ^ (lane & 15)) * 16; };
  struct Frag {
    bf16x8_t a[4], b[4];
  };
  // NF4_T: B tile nt of substep ks from the k-major slot, 4 K values per
  // transpose read
  auto trb = [&](const uint8_t* sb, int ks, int nt) -> bf16x8_t {
    typedef short s16x4_t __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4_t* lds_s16x4_t;
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)(lds_ptr_t)(sb + tboff[0][nt] + ks * 8192));
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)(lds_ptr_t)(sb + tboff[1][nt] + ks * 8192));
    typedef short s16x8_t __attribute__((ext_vector_type(8)));
    const s16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, v);
  };
  // (B in the k-major NF4_T layout when bt, else in the DMA layout)
  auto load_frag_at = [&](Frag& f, const uint8_t* sa, const uint8_t* sb, int ks, bool bt) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) f.a[mt] = *(const bf16x8_t*)(sa + fq + mt * 256 + fpos(ks));
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      if (NT && bt) f.b[nt] = trb(sb, ks, nt);
      else f.b[nt] = *(const bf16x8_t*)(sb + gq + nt * 256 + fpos(ks));
    }
  };
  auto load_frag = [&](Frag& f, int st, int ks) { load_frag_at(f, slot(2 * st), slot(2 * st + 1), ks, true); };
  auto mma = [&](const Frag& f) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[mt], f.b[nt], acc[mt][nt], 0, 0, 0);
  };
  // scheduling hint for one 16-MFMA substep: the fragment reads go with the
  // first 8 MFMAs, the loads (which write LDS, so they stay after the reads
  // in program order) with the last 8
  auto interleave = [&](int nds, int nvm) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < nds) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < nvm) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
    }
  };

  const bool rp_on = (EPI == EPI_GATEUP || EPI == EPI_ACT_BWD) && p.rp_r > 0;
  // ACT_BWD: g and u of one epilogue slab, fetched a slab ahead (the first
  // beside the last k-step, or with an NF4 B before the K-extension) so that
  // their latency overlaps other work. Lane:
  // 8 consecutive columns of staged rows q * 4 + lane / 16, i.e. tile rows
  // wm*128 + 8*((lane/16) >> 1) + 2*mt + ((lane/16) & 1) + 16 q; rows past M
  // and columns past N read nothing (zeros).
  u32x4_t gw[8], uw[8];
  auto fetch_gu = [&](int mt, auto in_c) {
    constexpr bool IN = decltype(in_c)::value;
    const int sl = lane >> 4;
    const int row0 = m0 + wm * 128 + 8 * (sl >> 1) + 2 * mt + (sl & 1);
    const int col = n0 + wn * 128 + (lane & 15) * 8;
    const int64_t o0 = (int64_t)row0 * p.hdim + col;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      gw[q] = u32x4_t{0u, 0u, 0u, 0u};
      uw[q] = u32x4_t{0u, 0u, 0u, 0u};
      if (IN || (row0 + 16 * q < p.M && col < p.N)) {
        const int64_t o = o0 + (int64_t)(16 * q) * p.hdim;
        gw[q] = *(const u32x4_t*)(p.g_in + o);
        uw[q] = *(const u32x4_t*)(p.u_in + o);
      }
    }
  };
  // GATEUP row product: the rank-r fragments of the wave's 64 H columns
  // (registers), waited for before the epilogue: waited for behind its
  // conditional stores, they would cost a wait for all of those.
  bf16x8_t rpb[2];
  auto load_rpb = [&]() {
    const int jr = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const int64_t c = (int64_t)((n0 + wn * 128) >> 1) + 32 * kc + 8 * kq;
      rpb[kc] = bf16x8_t{};
      if (jr < p.rp_r && c < p.hdim) rpb[kc] = *(const bf16x8_t*)(p.rp_l + (int64_t)jr * p.rp_ldl + c);
    }
  };
  // ACT_BWD row product: the rank-r operand over the tile's 256 columns
  // (gate rows 0-15, then up rows 16-31: 32 x 256 bf16) is brought by DMA
  // into the end of ring slot 4, which the epilogue's staging leaves alone;
  // the epilogue reads it from LDS. Row i keeps logical 16-byte chunk c at
  // physical chunk c ^ (i & 15) of its 512 bytes: the 16 rows of a fragment
  // read hit 16 different bank groups. Rows j >= rp_r and columns at or past
  // hdim load as zeros.
  constexpr int RPL_OFF = 5 * G_SLOT - 16384;
  auto issue_rpl = [&]() {
    const int up = wave >= 2;   // waves 0, 1: gate rows; 2, 3: up rows
    const uint64_t base = (uint64_t)(up ? p.rp_l2 : p.rp_l);
    const int nrec = rec_bytes(p.rp_r, p.rp_ldl);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int inst = 4 * wave + q;
      const int i = 2 * inst + (lane >> 5), j = i & 15;
      const int c = (lane & 31) ^ j;
      const int64_t col = n0 + 8 * c;
      const bool in = j < p.rp_r && col < p.hdim;
      bload_lds<16>(base, nrec, smem + RPL_OFF + inst * 1024,
                    in ? (uint32_t)((int64_t)j * p.rp_ldl + col) * 2u : OOB, 0);
    }
  };
  // The bf16 B path loads the tile's tail operands beside its last step's
  // MFMAs, when ring slots f, f+1, f+2 (mod 5, f = 2 ns for ns steps) are
  // free (the last step reads the other two): the K-extension's first step
  // goes to slots ka, kb, ACT_BWD's rank-r operand to slot 4 if that is free
  // and not one of them, the row-product operands and g/u to registers.
  constexpr bool tail_pre = !NF4;
  const int tail_f = tail_pre ? (2 * (kt1 - kt0)) % 5 : 0;
  const bool rpl_pre = tail_pre && EPI == EPI_ACT_BWD && rp_on && tail_f >= 2;
  const int ka = rpl_pre && tail_f == 4 ? 1 : tail_f;
  const int kb = rpl_pre && tail_f == 3 ? 0 : (tail_f + 1) % 5;
  // ---- main loop ----
  // Step s frees the slots of step s-1, so it issues H_2s+3 (B of step s+1,
  // for s >= 1: the prologue has B of step 1) over its first two substeps and
  // H_2s+4 (A of step s+2) over its second and third, then waits for step
  // s+1's A and B; A of step s+2, issued last, may stay in flight (vmcnt
  // retires in order).
  const int ns = kt1 - kt0, nh = 2 * ns;
  if constexpr (NF4) {
    // NF4 B operand. The B half-stage of step s+1 goes to the slot of A of
    // step s-1, free from the barrier that ends step s-1's third substep; it
    // is dequantized from there (the fourth substep of step s-1) through the
    // third substep of step s, i.e. beside 64 MFMAs. Codes of step s+2 are
    // waited for, copied out and the codes of step s+3 issued in that fourth
    // substep of step s: a full step of latency. A of step s+2 is loaded in
    // the first two substeps of step s, as for bf16 B. Load order per step:
    // A[0-3], A[4-7], codes; so the end of step s waits for A of s+1 with the
    // codes of s+2 and A of s+2 behind it, and the fourth substep waits for
    // the codes of s+2 with A of s+2 behind them.
    QRegs cq, wq;
    uint32_t P[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u}, D[8];
    auto bslot = [&](int s_) { return slot(2 * s_ + 1); };
    // the codes in cq have landed: move them to wq and issue step kt's into
    // cq (if `next`). The moves are explicit (early-clobber outputs), so that
    // wq never shares registers with cq: the loads into cq then reuse cq's
    // registers and nothing in flight is copied at the loop's back edge.
    auto take_q = [&](int kt, auto next_c) {
#pragma unroll
      for (int i = 0; i < 8; ++i) asm volatile("v_mov_b32 %0, %1" : "=&v"(wq.c[i]) : "v"(cq.c[i]));
      asm volatile("v_mov_b32 %0, %1" : "=&v"(wq.a[0]) : "v"(cq.a[0]));
      if constexpr (decltype(next_c)::value) issue_q(kt, cq);
    };
    auto table_all = [&]() {
#pragma unroll
      for (int t = 0; t < 6; ++t) qtable_part(t, wq, D, P);
    };
    // MFMA q of a substep: tile (q / 4, q % 4)
    auto mma_ab = [&](const bf16x8_t (&fa)[4], const bf16x8_t (&fb)[4], int q) {
      acc[q >> 2][q & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[q >> 2], fb[q & 3], acc[q >> 2][q & 3], 0, 0, 0);
    };
    // fragment tile idx of A (idx 0-3) or of row-major B (idx 4-7), substep ks of step st
    auto frag1 = [&](Frag& f, int st, int ks, int idx) {
      if (idx < 4) f.a[idx] = *(const bf16x8_t*)(slot(2 * st) + fq + idx * 256 + fpos(ks));
      else f.b[idx - 4] = *(const bf16x8_t*)(slot(2 * st + 1) + gq + (idx - 4) * 256 + fpos(ks));
    };
    using T_ = std::integral_constant<bool, true>;
    using F_ = std::integral_constant<bool, false>;
    if constexpr (!NT) {
    // Prologue, branch-free: the loads of steps 1 and 2 are issued even when
    // the job has fewer steps (they then read rows past the end, or zeros,
    // into slots nothing reads), so every path reaches the loop with the
    // same loads in flight.
#pragma unroll
    for (int j = 0; j < 8; ++j) issue_half(0, j);
    issue_q(kt0, cq);
#pragma unroll
    for (int j = 0; j < 4; ++j) issue_half(2, j);
    wait_vmem<4>();
    take_q(kt0 + 1, std::true_type());
    table_all();
#pragma unroll
    for (int j = 4; j < 8; ++j) issue_half(2, j);
    {
      QStep S0;
#pragma unroll
      for (int pp = 0; pp < NPART; ++pp) qpart(S0, pp, wq, P, bslot(0));
    }
    wait_vmem<4>();   // codes of step 1 (A[4-7] of step 1 behind them)
    take_q(kt0 + 2, std::true_type());
    table_all();
    QStep S;   // the dequant state of the B half-stage in progress, across steps
#pragma unroll
    for (int pp = 0; pp < NPRE; ++pp) qpart(S, pp, wq, P, bslot(1));
    wait_vm<4 + NQ>();
    ring_barrier();
    Frag f0, f1;
    load_frag(f0, 0, 0);
    // Step st, with the order of its instructions fixed: each MFMA is followed
    // by its share of the other work. Substeps 0-2 finish B of step st+1 (its
    // last NPART - NPRE parts, one per MFMA) in the slot of A of step st-1,
    // read the next substep's fragments (one after each of the first 8 MFMAs)
    // and load A of step st+2 (substeps 0-1, after MFMAs 8-11). Substep 3
    // (after the barrier) takes the codes of step st+2, issues those of step
    // st+3, forms the table for B of step st+2 and does that B's first NPRE
    // parts (its slot, that of A of step st, is free from the barrier on).
    // b1: B of step st+1 to write (st+1 < ns); b2: codes of step st+2 to take
    // and A of step st+2 to load (st+2 < ns); c3: codes of step st+3 to load.
    auto stepq = [&](int st, auto b1_c, auto b2_c, auto c3_c) {
      constexpr bool b1 = decltype(b1_c)::value, b2 = decltype(b2_c)::value;
      uint8_t* sb = bslot(st + 1);
#pragma unroll
      for (int ss = 0; ss < 3; ++ss) {
        Frag& cur = (ss & 1) ? f1 : f0;
        Frag& nxt = (ss & 1) ? f0 : f1;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          mma_ab(cur.a, cur.b, i);
          __builtin_amdgcn_sched_barrier(0);
          if (i < 8) frag1(nxt, st, ss + 1, i);
          if (b2 && ss < 2 && i >= 8 && i < 12) issue_half(2 * st + 4, 4 * ss + i - 8);
          if (b1) qpart(S, NPRE + 16 * ss + i, wq, P, sb);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (b1) {
        if (b2) wait_vm<NQ + 8>(); else wait_vm<0>();
      }
      ring_barrier();
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        mma_ab(f1.a, f1.b, i);
        __builtin_amdgcn_sched_barrier(0);
        if (b1 && i < 8) frag1(f0, st + 1, 0, i);
        if (b2) {
          if (i == 1) take_q(kt0 + st + 3, c3_c);
          if (i >= 2 && i < 8) qtable_part(i - 2, wq, D, P);
          if (i >= 8) qpart(S, i - 8, wq, P, bslot(st + 2));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    int st = 0;
    for (; st < ns - 3; ++st) stepq(st, T_(), T_(), T_());
    if (ns >= 3) stepq(st++, T_(), T_(), F_());
    if (ns >= 2) stepq(st++, T_(), F_(), F_());
    stepq(st, F_(), F_(), F_());
    } else {
    // Transposed B. The compiler waits for every LDS-DMA load in flight before
    // an LDS transpose read (it cannot tell which LDS bytes they write), so
    // all of a step's B fragments (16 tiles, 32 transpose reads) are read in
    // the fourth substep of the step before, right after its barrier, when no
    // DMA is in flight; A of step s+2 is loaded after them, at the end of
    // that substep, and waited for at the end of step s+1. The codes of step
    // s+3 are issued at its start, ahead of that A.
    bf16x8_t tb[4][4];      // B fragments of the current step [substep][tile]
    bf16x8_t fa0[4], fa1[4];
    auto afrag = [&](bf16x8_t (&fa)[4], int st, int ks, int mt) {
      fa[mt] = *(const bf16x8_t*)(slot(2 * st) + fq + mt * 256 + fpos(ks));
    };
    // prologue (branch-free, as row-major): A of steps 0, 1 and the codes of
    // step 0; B of step 0 dequantized; its fragments read; the codes of step
    // 1 taken, those of step 2 issued; A of step 2 issued.
#pragma unroll
    for (int j = 0; j < 8; ++j) issue_half(0, j);
    issue_q(kt0, cq);
#pragma unroll
    for (int j = 0; j < 8; ++j) issue_half(2, j);
    wait_vm<0>();
    take_q(kt0 + 1, std::true_type());
    table_all();
    {
      QStep S0;
#pragma unroll
      for (int pp = 0; pp < NPART; ++pp) qpart(S0, pp, wq, P, bslot(0));
    }
    wait_vm<NQ>();
    ring_barrier();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) tb[ks][nt] = trb(bslot(0), ks, nt);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) afrag(fa0, 0, 0, mt);
    take_q(kt0 + 2, std::true_type());
    table_all();
    QStep S;   // the dequant state of the B half-stage in progress, across steps
#pragma unroll
    for (int pp = 0; pp < NPRE; ++pp) qpart(S, pp, wq, P, bslot(1));
#pragma unroll
    for (int j = 0; j < 8; ++j) issue_half(4, j);
    auto stepq_t = [&](int st, auto b1_c, auto b2_c, auto c3_c) {
      constexpr bool b1 = decltype(b1_c)::value, b2 = decltype(b2_c)::value;
      uint8_t* sb = bslot(st + 1);
#pragma unroll
      for (int ss = 0; ss < 3; ++ss) {
        bf16x8_t (&cur)[4] = (ss & 1) ? fa1 : fa0;
        bf16x8_t (&nxt)[4] = (ss & 1) ? fa0 : fa1;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          mma_ab(cur, tb[ss], i);
          __builtin_amdgcn_sched_barrier(0);
          if (i < 4) afrag(nxt, st, ss + 1, i);
          if (b1) qpart(S, NPRE + 16 * ss + i, wq, P, sb);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (b1) wait_vm<0>();   // A of step st+1 (the codes of step st+2, older, too)
      ring_barrier();
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        mma_ab(fa1, tb[3], i);
        __builtin_amdgcn_sched_barrier(0);
        if (b1) {
          if (b2 && i == 0) take_q(kt0 + st + 3, c3_c);
          // fragments of step st+1: tiles of substeps 0-2 two reads per MFMA,
          // those of substep 3 each after the last MFMA that reads its register
          if (i < 12) tb[i >> 2][i & 3] = trb(sb, i >> 2, i & 3);
          else tb[3][i - 12] = trb(sb, 3, i - 12);
          if (i < 4) afrag(fa0, st + 1, 0, i);
          if (b2 && i >= 1 && i < 7) qtable_part(i - 1, wq, D, P);
          if (b2 && i >= 8) qpart(S, i - 8, wq, P, bslot(st + 2));
        }
        if (b2 && i == 15) {
#pragma unroll
          for (int j = 0; j < 8; ++j) issue_half(2 * st + 4, j);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    int st = 0;
    for (; st < ns - 3; ++st) stepq_t(st, T_(), T_(), T_());
    if (ns >= 3) stepq_t(st++, T_(), T_(), F_());
    if (ns >= 2) stepq_t(st++, T_(), F_(), F_());
    stepq_t(st, F_(), F_(), F_());
    }
  } else {
  for (int i = 0; i < 4 && i < nh; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) issue_half(i, j);
  }
  if (nh > 2) wait_vm<16>(); else wait_vm<0>();
  ring_barrier();
  Frag f0, f1;
  load_frag(f0, 0, 0);
  auto step = [&](int st, auto ib_c, auto ia_c) {
    constexpr bool iB = decltype(ib_c)::value, iA = decltype(ia_c)::value;
#pragma unroll
    for (int ks = 0; ks < 3; ++ks) {
      Frag& cur = (ks & 1) ? f1 : f0;
      Frag& nxt = (ks & 1) ? f0 : f1;
      load_frag(nxt, st, ks + 1);
      // B of step st+1: loads 0-5 in substep 0, 6-7 in substep 1; A of step
      // st+2: loads 0-1 in substep 1, 2-7 in substep 2 (spread, B first)
      const int b0 = ks == 0 ? 0 : (ks == 1 ? 6 : 8), b1 = ks == 0 ? 6 : 8;
      const int a0 = ks == 1 ? 0 : (ks == 2 ? 2 : 8), a1 = ks == 1 ? 2 : (ks == 2 ? 8 : 0);
      if (iB) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (j >= b0 && j < b1) issue_half(2 * st + 3, j);
      }
      if (iA) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (j >= a0 && j < a1) issue_half(2 * st + 4, j);
      }
      mma(cur);
      interleave(8, (iB ? b1 - b0 : 0) + (iA && a1 > a0 ? a1 - a0 : 0));
      __builtin_amdgcn_sched_barrier(0);
    }
    if (st + 1 < ns) {
      if (iA) wait_vm<8>(); else wait_vm<0>();
    }
    ring_barrier();
    if (st + 1 < ns) load_frag(f0, st + 1, 0);
    mma(f1);
    interleave(8, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  // the tile's tail operands, beside the last step's MFMAs
  auto tail = [&]() {
    if (p.KE > 0 && ksp == 0) {   // the K-extension's first step, as the K-extension loop lays it out
      const uint64_t eA = (uint64_t)(p.Ae + (int64_t)m0 * p.ldae), eB = (uint64_t)(p.Be + (int64_t)n0 * p.ldbe);
      const int neA = rec_bytes(rowsA, p.ldae);
      const int neB = rec_bytes(rowsB, p.ldbe);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = drow(j), c = dcol(j);
        const bool in = c < p.KE;
        bload_lds<16>(eA, neA, slot(ka) + (8 * wave + j) * 1024, in ? (uint32_t)(row * p.ldae + c) * 2u : OOB, 0);
        bload_lds<16>(eB, neB, slot(kb) + (8 * wave + j) * 1024, in ? (uint32_t)(row * p.ldbe + c) * 2u : OOB, 0);
      }
    }
    if (rpl_pre) issue_rpl();
    if (EPI == EPI_GATEUP && rp_on) load_rpb();
    if (EPI == EPI_ACT_BWD) {
      if (interior) fetch_gu(0, std::integral_constant<bool, true>());
      else fetch_gu(0, std::integral_constant<bool, false>());
    }
  };
  using T_ = std::integral_constant<bool, true>;
  using F_ = std::integral_constant<bool, false>;
  if (ns >= 3) {
    step(0, F_(), T_());
    for (int st = 1; st < ns - 2; ++st) step(st, T_(), T_());
    step(ns - 2, T_(), F_());
    tail();
    step(ns - 1, F_(), F_());
  } else if (ns == 2) {
    step(0, F_(), F_());
    tail();
    step(1, F_(), F_());
  } else {
    tail();
    step(0, F_(), F_());
  }
  }   // bf16 B
  if (!tail_pre && EPI == EPI_GATEUP && rp_on) load_rpb();
  __builtin_amdgcn_sched_barrier(0);
  wait_vm<0>();
  __syncthreads();

  if (EPI == EPI_ACT_BWD && rp_on && !rpl_pre) issue_rpl();
  if (EPI == EPI_ACT_BWD && !tail_pre) {
    if (interior) fetch_gu(0, std::integral_constant<bool, true>());
    else fetch_gu(0, std::integral_constant<bool, false>());
  }

  // ---- K-extension ----
  // Two slot pairs take turns, so that step e+1 loads while step e multiplies:
  // pair 0 is where the bf16 path put step 0 (ka, kb), pair 1 the first two
  // other slots (not slot 4 while it holds dH's rank-r operand).
  if (p.KE > 0 && ksp == 0) {
    const uint64_t eA = (uint64_t)(p.Ae + (int64_t)m0 * p.ldae), eB = (uint64_t)(p.Be + (int64_t)n0 * p.ldbe);
    const int neA = rec_bytes(rowsA, p.ldae);
    const int neB = rec_bytes(rowsB, p.ldbe);
    auto issue_ke = [&](int e, uint8_t* sa, uint8_t* sb) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = drow(j), c = e * BK + dcol(j);   // c < KE covers all 8 columns (KE % 16 == 0)
        const bool in = c < p.KE;
        bload_lds<16>(eA, neA, sa + (8 * wave + j) * 1024, in ? (uint32_t)(row * p.ldae + c) * 2u : OOB, 0);
        bload_lds<16>(eB, neB, sb + (8 * wave + j) * 1024, in ? (uint32_t)(row * p.ldbe + c) * 2u : OOB, 0);
      }
    };
    const int p0a = tail_pre ? ka : 0, p0b = tail_pre ? kb : 1;
    int p1a = -1, p1b = -1;
    for (int i = 0; i < 5; ++i) {
      if (i == p0a || i == p0b || (EPI == EPI_ACT_BWD && rp_on && i == 4)) continue;
      if (p1a < 0) p1a = i;
      else if (p1b < 0) p1b = i;
    }
    const int nke = (p.KE + BK - 1) / BK;
    if (!tail_pre) issue_ke(0, slot(p0a), slot(p0b));
    for (int e = 0; e < nke; ++e) {
      const bool odd = e & 1;
      if (e + 1 < nke) {   // its pair was last read before the previous barrier
        issue_ke(e + 1, slot(odd ? p0a : p1a), slot(odd ? p0b : p1b));
        wait_vm<16>();     // all but step e+1's 16 loads per wave
      } else {
        wait_vm<0>();
      }
      ring_barrier();
      const int nsub = (min(BK, p.KE - e * BK) + 15) >> 4;
      const uint8_t* sa = slot(odd ? p1a : p0a);
      const uint8_t* sb = slot(odd ? p1b : p0b);
      for (int ks = 0; ks < nsub; ++ks) {
        Frag f;
        load_frag_at(f, sa, sb, ks, false);
        mma(f);
      }
      ring_barrier();
    }
  }

  if (EPI == EPI_ACT_BWD && rp_on) {
    wait_vm<0>();
    __syncthreads();
  }

  // ---- epilogue ----
  // acc[mt][nt][v]: MFMA row r = 8*(v/4) + 4*(lane/32) + v%4, col j = lane%32, i.e.
  // tile row wm*128 + 8*(r&15) + 2*mt + (r>>4), tile col wn*128 + 8*(j&15) + 2*nt + (j>>4).
  // Slab mt (32 rows) is staged through LDS as staged row s = 2*(r&15) + (r>>4)
  // (tile row wm*128 + 8*(s>>1) + 2*mt + (s&1)) by 128 columns. A lane writes
  // its four nt values of one row as one 16-byte store, so within each group
  // of 8 columns position 4*(j>>4) + nt holds tile column 2*nt + (j>>4):
  // tile column 2e + t of a group is element e of the group's first (t = 0)
  // or second (t = 1) 16 bytes. Readers restore tile order in registers.
  constexpr int SP = 132;  // floats per staged row
  float* stage = reinterpret_cast<float*>(smem) + wave * (32 * SP);
  const int col0 = n0 + wn * 128;
  // Row product (rp_r > 0). A slab's bf16 results (GATEUP: H, 32 x 64; ACT_BWD:
  // dg | du, 32 x 256) replace the first bytes of their own staged row once
  // the row has been read (one wave reads and writes it, and LDS serves a
  // wave in order). The 528-byte row pitch is 33 16-byte units, so the 16
  // rows of a fragment read hit 16 different bank groups. The panel is
  // multiplied by the rank-r operand on MFMA 16x16x32, and the four 16x16
  // results per lane and slab are parked in LDS after the staging regions:
  // xpark[slab][wave][t] (t = 2 half + rg, 64 lanes x 16 bytes each). At the
  // end of the tile the two waves of a tile row add their halves of the
  // columns and store one fp32 partial per tile column.
  constexpr int PP = 2 * SP;   // bf16 per panel row
  constexpr int ND = EPI == EPI_GATEUP ? 2 : 4;
  f32x4_t* xpark = reinterpret_cast<f32x4_t*>(smem + 4 * 32 * SP * 4);
  // ACT_BWD: the rank-r fragments of this wave's 128 columns from the LDS
  // copy (half 0: gate rows, 1: up rows); lane (i = lane % 16, q = lane / 16)
  // gets row i, columns 32 kc + 8 q of the wave's range
  auto lds_frags = [&](bf16x8_t* b, int half) {
    const int ln = lane_here(), jr = ln & 15, kq = ln >> 4;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const int c = wn * 16 + 4 * kc + kq;
      b[kc] = *(const bf16x8_t*)(smem + RPL_OFF + (16 * half + jr) * 512 + ((c ^ jr) << 4));
    }
  };
  // D[j][s] = sum_c L[j][c] panel[s][c] over the wave's panel columns for the
  // 32 panel rows (L as the row operand); lane (sr, kq) gets j = 4 kq + v of
  // panel row 16 rg + sr in d[rg][v]; parked as xpark[mt][wave][2 half + rg]
  auto rowprod = [&](const uint16_t* pan, auto nkc_c, const bf16x8_t* b, int mt, int half) {
    constexpr int NKC = decltype(nkc_c)::value;
    const int ln = lane_here(), sr = ln & 15, kq = ln >> 4;
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      f32x4_t d = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const bf16x8_t a = *(const bf16x8_t*)(pan + (16 * rg + sr) * PP + 32 * kc + 8 * kq);
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[kc], a, d, 0, 0, 0);
      }
      xpark[((mt * 4 + wave) * ND + 2 * half + rg) * 64 + ln] = d;
    }
  };
  // after the four slabs: wave (wm, wn) sums and stores slabs 2 wn and 2 wn + 1
  // of its tile row, adding the wn = 0 half of the columns first
  auto rowprod_store = [&]() {
    const int rw = EPI == EPI_GATEUP ? p.rp_r : 2 * p.rp_r;
    const int ln = lane_here(), sr = ln & 15, j0 = 4 * (ln >> 4);
    float* out = p.rp_part + (int64_t)tn * p.M * rw;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int mt = 2 * wn + k;
#pragma unroll
      for (int t = 0; t < ND; ++t) {
        const int half = t >> 1, rg = t & 1;
        const f32x4_t d = xpark[((mt * 4 + 2 * wm) * ND + t) * 64 + ln] +
                          xpark[((mt * 4 + 2 * wm + 1) * ND + t) * 64 + ln];
        const int s = 16 * rg + sr;
        const int row = m0 + wm * 128 + 8 * (s >> 1) + 2 * mt + (s & 1);
        const int jofs = half * p.rp_r;
        if (row >= p.M || j0 >= p.rp_r) continue;
        float* o = out + (int64_t)row * rw + jofs + j0;
        if (((jofs | rw) & 3) == 0 && j0 + 4 <= p.rp_r) {
          *(f32x4_t*)o = d;
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (j0 + v < p.rp_r) o[v] = d[v];
        }
      }
    }
  };

  // one slab per call; mt is a compile-time constant so that acc stays in registers
  auto slab = [&](auto mt_c, auto act_c, auto in_c) {
    constexpr int mt = decltype(mt_c)::value;
    constexpr int ACT = decltype(act_c)::value;
    constexpr bool IN = decltype(in_c)::value;
    auto grow = [&](int s) { return m0 + wm * 128 + 8 * (s >> 1) + 2 * mt + (s & 1); };
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3), j = lane & 31;
      *(f32x4_t*)&stage[(2 * (r & 15) + (r >> 4)) * SP + 8 * (j & 15) + 4 * (j >> 4)] =
          f32x4_t{acc[mt][0][v], acc[mt][1][v], acc[mt][2][v], acc[mt][3][v]};
    }
    wave_sync();   // the staging region is this wave's own
    if (EPI == EPI_STORE || EPI == EPI_STORE3 || EPI == EPI_ACT_BWD) {
      // lane: 8 consecutive columns of one staged row; 4 rows per pass.
      // Staged row q * 4 + lane / 16 is tile row row0 + 16 q, so every output
      // offset is the one of pass 0 plus q times a uniform stride.
      const int cc = (lane & 15) * 8;
      const int row0 = grow(lane >> 4), col = col0 + cc;
      uint16_t* cbase = p.C;
      int64_t cld = p.ldc, ccol = col;
      if (EPI == EPI_STORE3) {   // the 8 columns lie in one output (nc1, nc2 multiples of 8)
        if (col >= p.nc2) { cbase = p.C2; cld = p.ldc2; ccol = col - p.nc2; }
        else if (col >= p.nc1) { cbase = p.C1; cld = p.ldc1; ccol = col - p.nc1; }
      }
      const int64_t coff0 = (int64_t)row0 * cld + ccol;
      const int64_t poff0 = ((int64_t)ksp * p.M + row0) * p.N + col;
      const int64_t doff0 = (int64_t)row0 * (2 * p.hdim) + col;
      const bool colok = col < p.N;
      // one output row segment from its staged values x0 | x1
      auto emit = [&](int q, const f32x4_t x0, const f32x4_t x1, auto split_c) {
        constexpr bool SPLIT = decltype(split_c)::value;
        const int s = q * 4 + (lane >> 4);
        const int row = row0 + 16 * q;
        u32x4_t odg = u32x4_t{0u, 0u, 0u, 0u}, odu = u32x4_t{0u, 0u, 0u, 0u};
        if (IN || (row < p.M && colok)) {
          if ((EPI == EPI_STORE || EPI == EPI_STORE3) && SPLIT) {   // fp32 partial
            float* o = p.part + poff0 + (int64_t)(16 * q) * p.N;
            *(f32x4_t*)o = f32x4_t{x0[0], x1[0], x0[1], x1[1]};
            *(f32x4_t*)(o + 4) = f32x4_t{x0[2], x1[2], x0[3], x1[3]};
          } else if (EPI == EPI_STORE || EPI == EPI_STORE3) {
            u32x4_t o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(x0[e], x1[e]);
            *(u32x4_t*)(cbase + coff0 + (int64_t)(16 * q) * cld) = o;
          } else {  // staged values are dH
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float dg[2], du[2];
#pragma unroll
              for (int t = 0; t < 2; ++t) {
                const float g = bf16_to_f32(t ? (gw[q][e] >> 16) : (gw[q][e] & 0xFFFFu));
                const float u = bf16_to_f32(t ? (uw[q][e] >> 16) : (uw[q][e] & 0xFFFFu));
                float a, da;
                act_fwd_bwd_t<ACT>(g, &a, &da);
                const float d = t ? x1[e] : x0[e];
                dg[t] = d * u * da;
                du[t] = d * a;
              }
              odg[e] = pack_bf16x2(dg[0], dg[1]);
              odu[e] = pack_bf16x2(du[0], du[1]);
            }
            const int64_t od = doff0 + (int64_t)(16 * q) * (2 * p.hdim);
            *(u32x4_t*)(p.dgu + od) = odg;
            *(u32x4_t*)(p.dgu + od + p.hdim) = odu;
          }
        }
        if (EPI == EPI_ACT_BWD && rp_on) {   // over the row just read; zeros outside the output
          uint16_t* pr = reinterpret_cast<uint16_t*>(stage) + s * PP + cc;
          *(u32x4_t*)pr = odg;
          *(u32x4_t*)(pr + 128) = odu;
        }
      };
      // the staged values of QG rows are read before any of them is used, so
      // that the LDS latency is waited for once per group instead of per row
      // (a row's row-product bf16 overwrite comes after its group's reads)
      auto rows = [&](auto split_c) {
        constexpr int QG = EPI == EPI_ACT_BWD ? 4 : 8;
#pragma unroll
        for (int qg = 0; qg < 8; qg += QG) {
          f32x4_t xs[QG][2];
#pragma unroll
          for (int i = 0; i < QG; ++i) {
            const float* x = &stage[((qg + i) * 4 + (lane >> 4)) * SP + cc];
            xs[i][0] = *(const f32x4_t*)x;
            xs[i][1] = *(const f32x4_t*)(x + 4);
          }
#pragma unroll
          for (int i = 0; i < QG; ++i) emit(qg + i, xs[i][0], xs[i][1], split_c);
        }
      };
      if ((EPI == EPI_STORE || EPI == EPI_STORE3) && nsplit > 1)
        rows(std::integral_constant<bool, true>());
      else
        rows(std::integral_constant<bool, false>());
      // the next slab's g and u: this slab's are consumed
      if constexpr (EPI == EPI_ACT_BWD && mt < 3) fetch_gu(mt + 1, in_c);
      if (EPI == EPI_ACT_BWD && rp_on) {
        wave_sync();
        const uint16_t* pan = reinterpret_cast<const uint16_t*>(stage);
        bf16x8_t lb[4];
        lds_frags(lb, 0);
        rowprod(pan, std::integral_constant<int, 4>(), lb, mt, 0);
        lds_frags(lb, 1);
        rowprod(pan + 128, std::integral_constant<int, 4>(), lb, mt, 1);
      }
    } else {  // EPI_GATEUP: staged columns [gate j0..+31 | up j0..+31 | gate j0+32.. | up j0+32..]
      const int jj = (lane & 7) * 8;                       // 0..56: output index within 64
      const int gcol = (jj >> 5) * 64 + (jj & 31);         // staged gate column (up = +32)
      const int64_t j = (int64_t)(col0 >> 1) + jj;
      // staged row q * 8 + lane / 8 is tile row row0 + 32 q
      const int row0 = grow(lane >> 3);
      const int64_t hoff0 = (int64_t)row0 * p.hdim + j;
      // all four rows' staged values first: one LDS wait for the slab (a
      // row's H overwrite comes after every read)
      f32x4_t gx[4][2], ux[4][2];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float* gs = &stage[(q * 8 + (lane >> 3)) * SP + gcol];
        gx[q][0] = *(const f32x4_t*)gs;
        gx[q][1] = *(const f32x4_t*)(gs + 4);
        ux[q][0] = *(const f32x4_t*)(gs + 32);
        ux[q][1] = *(const f32x4_t*)(gs + 36);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int s = q * 8 + (lane >> 3);
        const int row = row0 + 32 * q;
        u32x4_t oh = u32x4_t{0u, 0u, 0u, 0u};
        if (IN || (row < p.M && col0 < p.N)) {
          const f32x4_t g0 = gx[q][0], g1 = gx[q][1];
          const f32x4_t u0 = ux[q][0], u1 = ux[q][1];
          float gv[8], uv[8];   // tile order
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            gv[2 * e] = g0[e];
            gv[2 * e + 1] = g1[e];
            uv[2 * e] = u0[e];
            uv[2 * e + 1] = u1[e];
          }
          u32x4_t og, ou;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            og[e] = pack_bf16x2(gv[2 * e], gv[2 * e + 1]);
            ou[e] = pack_bf16x2(uv[2 * e], uv[2 * e + 1]);
            // H from the rounded g and u (the values the backward reads)
            const float g0 = __uint_as_float(og[e] << 16), g1 = __uint_as_float(og[e] & 0xFFFF0000u);
            const float u0 = __uint_as_float(ou[e] << 16), u1 = __uint_as_float(ou[e] & 0xFFFF0000u);
            oh[e] = pack_bf16x2(act_fwd_t<ACT>(g0) * u0, act_fwd_t<ACT>(g1) * u1);
          }
          const int64_t o = hoff0 + (int64_t)(32 * q) * p.hdim;
          *(u32x4_t*)(p.g_out + o) = og;
          *(u32x4_t*)(p.u_out + o) = ou;
          *(u32x4_t*)(p.h_out + o) = oh;
        }
        if (rp_on)   // over the row just read; zeros outside the output
          *(u32x4_t*)(reinterpret_cast<uint16_t*>(stage) + s * PP + jj) = oh;
      }
      if (rp_on) {
        wave_sync();
        rowprod(reinterpret_cast<const uint16_t*>(stage), std::integral_constant<int, 2>(), rpb, mt, 0);
      }
    }
    wave_sync();
  };
  // the activation is fixed per launch: one branch here, none per value
  auto slabs = [&](auto act_c, auto in_c) {
    slab(std::integral_constant<int, 0>(), act_c, in_c);
    slab(std::integral_constant<int, 1>(), act_c, in_c);
    slab(std::integral_constant<int, 2>(), act_c, in_c);
    slab(std::integral_constant<int, 3>(), act_c, in_c);
  };
  auto slabs_in = [&](auto act_c) {
    // the three-output epilogue keeps one body: a second copy spills there
    if (EPI != EPI_STORE3 && interior) slabs(act_c, std::integral_constant<bool, true>());
    else slabs(act_c, std::integral_constant<bool, false>());
  };
  if ((EPI == EPI_GATEUP || EPI == EPI_ACT_BWD) && p.act != 0)
    slabs_in(std::integral_constant<int, 1>());
  else
    slabs_in(std::integral_constant<int, 0>());
  if (rp_on) {
    // every wave's parked results are in LDS (lgkmcnt(0)); the global stores
    // in flight are not waited for
    wait_vm<63>();
    ring_barrier();
    rowprod_store();
  }
}

// Split-K reduction: C = bf16(sum_s part[s]) in fixed order; a thread takes 8
// columns of one row. EPI_STORE3 routes the columns as the GEMM epilogue does.
template <int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs p) {
  const int64_t groups = (int64_t)p.M * (p.N / 8);
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= groups) return;
  const int row = (int)(e / (p.N / 8));
  const int col = (int)(e - (int64_t)row * (p.N / 8)) * 8;
  f32x4_t s0 = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, s1 = s0;
  for (int k = 0; k < p.splits; ++k) {
    const float* src = p.part + ((int64_t)k * p.M + row) * p.N + col;
    s0 += *(const f32x4_t*)src;
    s1 += *(const f32x4_t*)(src + 4);
  }
  u32x4_t o;
  o[0] = pack_bf16x2(s0[0], s0[1]);
  o[1] = pack_bf16x2(s0[2], s0[3]);
  o[2] = pack_bf16x2(s1[0], s1[1]);
  o[3] = pack_bf16x2(s1[2], s1[3]);
  uint16_t* dst;
  if (EPI == EPI_STORE3)
    dst = col < p.nc1   ? p.C + (int64_t)row * p.ldc + col
          : col < p.nc2 ? p.C1 + (int64_t)row * p.ldc1 + (col - p.nc1)
                        : p.C2 + (int64_t)row * p.ldc2 + (col - p.nc2);
  else
    dst = p.C + (int64_t)row * p.ldc + col;
  *(u32x4_t*)dst = o;
}

template <int EPI, bool SEGA, int BSRC = BSRC_BF16>
static hipError_t launch_bf16(const GemmArgs& a, hipStream_t stream) {
  const int ntm = (a.M + BM - 1) / BM, ntn = (a.N + BN - 1) / BN;
  const int nsplit = a.splits > 1 ? a.splits : 1;
  if (nsplit > 1) {
    const int nk = a.K / BK, kper = (nk + nsplit - 1) / nsplit;
    if ((EPI != EPI_STORE && EPI != EPI_STORE3) || !a.part || a.N % 8 || (nsplit - 1) * kper >= nk)
      return hipErrorInvalidValue;
  }
  gemm_bf16_kernel<EPI, SEGA, BSRC><<<dim3(ntm * ntn * nsplit), dim3(256), 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  if (EPI == EPI_STORE || EPI == EPI_STORE3) {
    const int64_t groups = (int64_t)a.M * (a.N / 8);
    splitk_reduce_kernel<EPI><<<dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, stream>>>(a);
  }
  return hipGetLastError();
}

int gemm_rowprod_splits(int N) { return (N + BN - 1) / BN; }

int gemm_splits(int M, int N, int K) {
  const int64_t tiles = (int64_t)((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int nk = K / BK;
  if (tiles <= 0 || tiles >= 256 || nk < 16) return 1;
  int sp = (int)(256 / tiles);
  if (sp > nk / 8) sp = nk / 8;
  if (sp > 8) sp = 8;
  while (sp > 1 && (sp - 1) * ((nk + sp - 1) / sp) >= nk) --sp;
  return sp < 1 ? 1 : sp;
}

template <int BSRC>
static hipError_t launch_b(const GemmArgs& a, hipStream_t stream) {
  if (BSRC == BSRC_BF16) {
    if (a.A1) {   // K-segmented A: only the plain store is instantiated
      if (a.epi != EPI_STORE || !a.A2 || a.ka1 % BK || a.ka2 % BK || a.ka1 > a.ka2 || a.ka2 > a.K)
        return hipErrorInvalidValue;
      return launch_bf16<EPI_STORE, true>(a, stream);
    }
    switch (a.epi) {
      case EPI_STORE: return launch_bf16<EPI_STORE, false>(a, stream);
      case EPI_GATEUP: return launch_bf16<EPI_GATEUP, false>(a, stream);
      case EPI_ACT_BWD: return launch_bf16<EPI_ACT_BWD, false>(a, stream);
      case EPI_STORE3:
        if (a.nc1 % 8 || a.nc2 % 8 || a.nc1 > a.nc2 || !a.C1 || !a.C2) return hipErrorInvalidValue;
        return launch_bf16<EPI_STORE3, false>(a, stream);
    }
    return hipErrorInvalidValue;
  }
  if (a.A1 || !a.codes0 || !a.absmax0 || a.N % 64 || a.K % BK) return hipErrorInvalidValue;
  if (BSRC == BSRC_NF4_PAIR && (!a.codes1 || !a.absmax1)) return hipErrorInvalidValue;
  if (BSRC == BSRC_NF4_T && a.ksplit > 0 && (a.ksplit % BK || a.ksplit >= a.K || !a.codes1 || !a.absmax1))
    return hipErrorInvalidValue;
  switch (a.epi) {
    case EPI_STORE: return launch_bf16<EPI_STORE, false, BSRC>(a, stream);
    case EPI_GATEUP: return launch_bf16<EPI_GATEUP, false, BSRC>(a, stream);
    case EPI_ACT_BWD: return launch_bf16<EPI_ACT_BWD, false, BSRC>(a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  switch (a.bsrc) {
    case BSRC_BF16: return launch_b<BSRC_BF16>(a, stream);
    case BSRC_NF4: return launch_b<BSRC_NF4>(a, stream);
    case BSRC_NF4_PAIR: return launch_b<BSRC_NF4_PAIR>(a, stream);
    case BSRC_NF4_T: return launch_b<BSRC_NF4_T>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace qlora
