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
// Two kernels share the arguments (GemmArgs) and the epilogues.
//
// gemm_bf16_kernel (B in bf16: a staged dequant, or 16-bit base weights):
// 256 x 256 output tile per workgroup of 4 waves (one per SIMD) laid out
// 2 x 2, each wave 128 x 128 = 4 x 4 MFMA 32x32x16 tiles (256 fp32
// accumulators per lane). K is walked in 64-wide steps. Operands reach LDS
// through buffer loads straight into LDS (one buffer resource per operand
// tile, so rows past M or N read as zeros), into a ring of five 32 KB
// half-stage slots (one operand of one step each): while a step reads two
// slots, the next step and a half are in flight. The 1 KB load blocks are
// unpadded and XOR-swizzled so that the ds_read_b128 fragment reads stay
// conflict-free; the MFMA row order is permuted to match and undone in the
// epilogue. Fragments of the next substep are read while the matrix cores
// work on the current one, and sched_group_barrier hints interleave the LDS
// reads and load issues with the MFMAs.
// Optional extras: A split along K into up to three matrices (dX = sum of
// dY_p W_p over separately stored dY_p), and an epilogue that writes column
// ranges to three outputs (q, k, v from one GEMM).
//
// gemm_nt_kernel (B as NF4 codes, dequantized in the tile): 256 x 256 tile
// per workgroup of 8 waves (2 per SIMD) laid out 2 x 4, each wave 128 x 64 =
// 4 x 2 MFMA 32x32x16 tiles. K is walked in 64-wide steps through a 2-deep
// bf16 LDS ring; LDS rows are 128 B with the 16-byte chunk index
// XOR-swizzled by (row >> 1) & 7. The feed carries the 4-bit codes and the
// fp32 absmax (8 KB + 1 KB per step instead of 32 KB of bf16), brought by
// direct-to-LDS loads (global_load_lds_dwordx4) two steps ahead into a
// 3-deep ring of their own; the block dequantizes the next step's codes in
// LDS, bf16_rne(fp32_rne(level[code] * absmax)) exactly as the standalone
// dequant, while its matrix cores work on the current step. BSRC_NF4_T reads
// the weight transposed (the backward dX = dY W): the tile's rows are input
// features, its K runs over output features, and the dequant writes the
// transposed bf16 tile.
//
// Epilogues (both kernels): each wave stages a 32-row slab of its
// accumulators through its own LDS region, so only wave-local ordering is
// needed, and stores 16 bytes per lane. The gated epilogues take the
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

constexpr int BM = 256, BN = 256, BK = 64, NTHR = 512;
constexpr int NSTAGE = 2;

// Per-stage LDS layout (bytes): A [256][64] bf16, B [256][64] bf16, then (NF4
// modes) the raw codes of the step (8 KB) and 256 fp32 absmax (+ a spare copy).
constexpr int A_BYTES = BM * BK * 2;
constexpr int B_BYTES = BN * BK * 2;
constexpr int C_BYTES = 8192;
constexpr int S_BYTES = 2048;
constexpr int STAGE_BF16 = A_BYTES + B_BYTES;
// NF4 modes: the raw codes and absmax of a k-step (C_BYTES + S_BYTES) have a
// ring of their own, 3 deep, so that they are fetched two steps ahead: they
// are needed in the middle of the step before theirs (for the dequant).
constexpr int RAW_BYTES = C_BYTES + S_BYTES;
constexpr int NRAW = 3;

// element offset of (row, 16-byte chunk) in a [rows][64] bf16 LDS tile
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * BK + ((chunk ^ ((row >> 1) & 7)) << 3);
}

__device__ __forceinline__ int xcd_remap(int pid, int n) {
  const int X = 8;
  int q = n / X, rmd = n % X;
  int xcd = pid % X, local = pid / X;
  return (xcd < rmd ? xcd * (q + 1) : rmd * (q + 1) + (xcd - rmd) * q) + local;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// 16 bytes per lane from global memory straight into LDS at base + 16*lane.
__device__ __forceinline__ void dma16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds_base, 16, 0, 0);
}
// 4 bytes per lane into LDS at base + 4*lane.
__device__ __forceinline__ void dma4(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds_base, 4, 0, 0);
}

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

__constant__ uint32_t c_nf4_levels_gemm[16] = {QLORA_NF4_LEVEL_BITS};

template <int BSRC, int EPI>
__global__ __launch_bounds__(NTHR)
void gemm_nt_kernel(GemmArgs p) {
  constexpr bool NF4 = BSRC != BSRC_BF16;
  constexpr int STAGE = STAGE_BF16;
  constexpr int RAW = NF4 ? NRAW * RAW_BYTES : 0;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NSTAGE * STAGE + RAW + (NF4 ? 64 : 0)];
  float* lut = reinterpret_cast<float*>(smem + NSTAGE * STAGE + RAW);  // NF4 only

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  if (NF4) {
    if (tid < 16) lut[tid] = __uint_as_float(c_nf4_levels_gemm[tid]);
  }

  const int ntm = (p.M + BM - 1) / BM, ntn = (p.N + BN - 1) / BN;
  const int pid = xcd_remap(blockIdx.x, ntm * ntn);
  const int GM = 8;
  const int per_group = GM * ntn;
  const int group = pid / per_group;
  const int first_m = group * GM;
  const int gsz = min(ntm - first_m, GM);
  const int tm = first_m + (pid % per_group) % gsz;
  const int tn = (pid % per_group) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;
  const int nk = p.K / BK;

  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // ---- per-lane DMA sources (row and swizzled chunk fixed; k advances) ----
  // A/B tile: wave w, instruction j fills LDS slots (w*4 + j)*64 + lane of the
  // [256][8 x 16 B] tile; slot -> (row, physical chunk) -> logical chunk.
  const uint16_t* srcA[4];
  const uint16_t* srcB[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int slot = (wave * 4 + j) * 64 + lane;
    const int row = slot >> 3, phys = slot & 7;
    const int chunk = phys ^ ((row >> 1) & 7);
    srcA[j] = p.A + (int64_t)min(m0 + row, p.M - 1) * p.lda + chunk * 8;
    if (!NF4) srcB[j] = p.B + (int64_t)min(n0 + row, p.N - 1) * p.ldb + chunk * 8;
  }
  // NF4 raw data of one k-step: 8 KB of codes + 256 absmax; wave w moves one
  // 1 KB piece of codes and one 256 B piece of absmax (waves 4-7 duplicate
  // the absmax pieces of waves 0-3 into a spare copy, so every wave issues
  // the same number of loads).
  //   BSRC_NF4 / _PAIR: codes piece = rows w*32 .. w*32+31 of the tile
  //     (32 B = 64 codes each), absmax = one value per tile row.
  //   BSRC_NF4_T: the tile's K runs over weight rows: codes piece = weight
  //     rows k0 + w*8 .. +7, 128 B each (the tile's 256 input features);
  //     absmax = 64 weight rows x 4 blocks of 64 input features.
  const uint8_t* srcC = nullptr;
  const float* srcS = nullptr;
  const uint8_t* srcC1 = nullptr;  // transposed mode: second stacked weight
  const float* srcS1 = nullptr;
  int64_t cstep = 0, sstep = 0;    // source advance per k-step (bytes / floats)
  if (NF4) {
    if (BSRC == BSRC_NF4_T) {
      // weight [Nw][Kw]: Nw = GEMM K (reduction) rows, Kw = GEMM N features
      const int64_t kw = p.N;
      const int crow = wave * 8 + (lane >> 3);                        // weight row in step
      const int ccol = min(n0 + (lane & 7) * 32, p.N - 32);           // first feature of the piece
      srcC = p.codes0 + (int64_t)crow * (kw >> 1) + (ccol >> 1);
      srcC1 = p.codes1 ? p.codes1 + (int64_t)crow * (kw >> 1) + (ccol >> 1) : nullptr;
      cstep = (int64_t)BK * (kw >> 1);
      const int srow = (wave & 3) * 16 + (lane >> 2);                 // weight row in step
      const int sblk = min((n0 >> 6) + (lane & 3), (p.N >> 6) - 1);   // 64-feature block
      srcS = p.absmax0 + (int64_t)srow * (kw >> 6) + sblk;
      srcS1 = p.absmax1 ? p.absmax1 + (int64_t)srow * (kw >> 6) + sblk : nullptr;
      sstep = (int64_t)BK * (kw >> 6);
    } else {
      const int r = wave * 32 + (lane >> 1);
      int gn = min(n0 + r, p.N - 1);
      const uint8_t* codes = p.codes0;
      const float* amax = p.absmax0;
      int64_t wrow = gn;
      if (BSRC == BSRC_NF4_PAIR) {
        const int which = (gn >> 5) & 1;
        wrow = (int64_t)((gn >> 6) << 5) + (gn & 31);
        codes = which ? p.codes1 : p.codes0;
        amax = which ? p.absmax1 : p.absmax0;
      }
      srcC = codes + wrow * (int64_t)(p.K >> 1) + (lane & 1) * 16;
      cstep = BK >> 1;
      const int r2 = (wave & 3) * 64 + lane;
      gn = min(n0 + r2, p.N - 1);
      codes = p.codes0;
      amax = p.absmax0;
      wrow = gn;
      if (BSRC == BSRC_NF4_PAIR) {
        const int which = (gn >> 5) & 1;
        wrow = (int64_t)((gn >> 6) << 5) + (gn & 31);
        amax = which ? p.absmax1 : p.absmax0;
      }
      srcS = amax + wrow * (int64_t)(p.K >> 6);
      sstep = 1;
    }
  }

  auto stage_ptr = [&](int kt) { return smem + (kt % NSTAGE) * STAGE; };
  auto raw_ptr = [&](int kt) { return smem + NSTAGE * STAGE + (kt % NRAW) * RAW_BYTES; };
  // NF4: codes and absmax of step kt into its raw slot (2 loads per wave)
  auto issue_raw = [&](int kt) {
    uint8_t* rw = raw_ptr(kt);
    const uint8_t* c = srcC;
    const float* sc = srcS;
    int kl = kt;
    if (BSRC == BSRC_NF4_T && p.ksplit > 0 && kt * BK >= p.ksplit) {
      c = srcC1;
      sc = srcS1;
      kl = kt - p.ksplit / BK;
    }
    dma16(c + kl * cstep, rw + wave * 1024);
    dma4(sc + kl * sstep, rw + C_BYTES + wave * 256);
  };
  // the bf16 operands of step kt (A; B too when it is not NF4): 4 or 8 loads per wave
  auto issue = [&](int kt) {
    uint8_t* st = stage_ptr(kt);
    const int k0 = kt * BK;
#pragma unroll
    for (int j = 0; j < 4; ++j) dma16(srcA[j] + k0, st + (wave * 4 + j) * 1024);
    if (!NF4) {
#pragma unroll
      for (int j = 0; j < 4; ++j) dma16(srcB[j] + k0, st + A_BYTES + (wave * 4 + j) * 1024);
    }
  };

  // NF4: dequantize the raw codes of a landed k-step into its bf16 B tile.
  auto dequant_stage = [&](int kt) {
    uint8_t* st = stage_ptr(kt);
    const uint8_t* cb = raw_ptr(kt);
    const float* sb = (const float*)(raw_ptr(kt) + C_BYTES);
    uint16_t* bt = (uint16_t*)(st + A_BYTES);
    if (BSRC != BSRC_NF4_T) {
      // thread t: tile row t/2, 32 weights (k half t&1) = chunks 4*(t&1) .. +3
      const int row = tid >> 1, half = tid & 1;
      const u32x4_t w = *(const u32x4_t*)(cb + row * 32 + half * 16);
      const float amax = sb[row];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        u32x4_t o;
        const uint32_t word = w[c];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const uint32_t byte = (word >> (8 * b)) & 0xFFu;
          o[b] = pack_bf16x2(lut[byte >> 4] * amax, lut[byte & 0xFu] * amax);
        }
        lds_store16(&bt[swz(row, half * 4 + c)], o);
      }
    } else {
      // thread t: tile rows (input features) f0 .. f0+3, f0 = 4*(t & 63),
      // K (weight rows) q0 .. q0+7, q0 = 8*(t >> 6). Codes of weight row q,
      // features f0..f0+3 are 2 bytes at q*128 + f0/2; absmax of (q, f0/64).
      const int f0 = 4 * (tid & 63), q0 = 8 * (tid >> 6);
      float w[8][4];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint32_t two = *(const uint16_t*)(cb + (q0 + q) * 128 + (f0 >> 1));
        const float amax = sb[(q0 + q) * 4 + (f0 >> 6)];
        w[q][0] = lut[(two >> 4) & 0xFu] * amax;   // byte 0 high nibble: feature f0
        w[q][1] = lut[two & 0xFu] * amax;          // byte 0 low nibble: f0 + 1
        w[q][2] = lut[(two >> 12) & 0xFu] * amax;  // byte 1 high nibble: f0 + 2
        w[q][3] = lut[(two >> 8) & 0xFu] * amax;   // byte 1 low nibble: f0 + 3
      }
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        u32x4_t o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(w[2 * e][f], w[2 * e + 1][f]);
        lds_store16(&bt[swz(f0 + f, q0 >> 3)], o);
      }
    }
  };

  // Fragments of one 16-wide K substep: 4 A (rows of the wave) + 2 B (columns).
  struct Frag {
    bf16x8_t a[4], b[2];
  };
  auto load_frag = [&](Frag& f, const uint8_t* st, int ks) {
    const uint16_t* sa = (const uint16_t*)st;
    const uint16_t* sb = (const uint16_t*)(st + A_BYTES);
    const int ch = 2 * ks + (lane >> 5);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      f.a[mt] = *(const bf16x8_t*)&sa[swz(wm * 128 + mt * 32 + (lane & 31), ch)];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
      f.b[nt] = *(const bf16x8_t*)&sb[swz(wn * 64 + nt * 32 + (lane & 31), ch)];
  };
  auto mma = [&](const Frag& f) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[mt], f.b[nt], acc[mt][nt], 0, 0, 0);
  };
  auto compute = [&](const uint8_t* st, int nsub) {
    for (int ks = 0; ks < nsub; ++ks) {
      Frag f;
      load_frag(f, st, ks);
      mma(f);
    }
  };

  // ---- main K loop: 2-deep ring, DMA of step kt+1 in flight during step kt ----
  // Iteration kt: issue step kt+1; (NF4) once its codes land, dequantize
  // them; the MFMAs of step kt run meanwhile, with the fragments of the next
  // substep (and, across the barrier, of step kt+1's first substep) loaded
  // ahead. The closing barrier publishes step kt+1 and retires step kt.
  // NF4 issue order inside step kt: A of kt+1 (4 loads), then codes and
  // absmax of kt+2 (2 loads). Mid-step the codes of kt+1 (issued a step
  // earlier, older than both) must have landed: wait_vm<4 + 2>; at the end
  // A of kt+1 must have: wait_vm<2> (the codes of kt+2 may still fly).
  if (NF4) {
    issue_raw(0);
    issue(0);
    if (nk > 1) issue_raw(1);
    if (nk > 1) wait_vm<2>(); else wait_vm<0>();
  } else {
    issue(0);
    wait_vm<0>();
  }
  ring_barrier();   // step 0 raw data (and lut) visible
  if (NF4) {
    dequant_stage(0);
    if (nk > 1) wait_vm<2>(); else wait_vm<0>();   // its LDS stores done (codes of step 1 may fly)
    ring_barrier();
  }
  Frag f0, f1;
  load_frag(f0, stage_ptr(0), 0);
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    const bool more2 = kt + 2 < nk;
    if (more) issue(kt + 1);
    if (NF4 && more2) issue_raw(kt + 2);
    const uint8_t* st = stage_ptr(kt);
    load_frag(f1, st, 1);
    __builtin_amdgcn_sched_barrier(0);
    mma(f0);
    __builtin_amdgcn_sched_barrier(0);
    load_frag(f0, st, 2);
    __builtin_amdgcn_sched_barrier(0);
    mma(f1);
    __builtin_amdgcn_sched_barrier(0);
    if (NF4 && more) {
      if (more2) wait_vm<6>(); else wait_vm<4>();   // codes + absmax of step kt+1 landed
      ring_barrier();  // ... for every wave
      dequant_stage(kt + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    load_frag(f1, st, 3);
    __builtin_amdgcn_sched_barrier(0);
    mma(f0);
    __builtin_amdgcn_sched_barrier(0);
    if (NF4 && more2) wait_vm<2>();   // step kt+1 landed (codes of kt+2 may fly); LDS done
    else wait_vm<0>();
    ring_barrier();
    load_frag(f0, stage_ptr(more ? kt + 1 : kt), 0);
    __builtin_amdgcn_sched_barrier(0);
    mma(f1);
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();

  // ---- K-extension (LoRA up-projection), bf16 both sides, via registers ----
  for (int e = 0; e * BK < p.KE; ++e) {
    const int c0 = e * BK;
    const int nch = min(BK, p.KE - c0) >> 3;
    uint16_t* sa = (uint16_t*)smem;
    uint16_t* sb = (uint16_t*)(smem + A_BYTES);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (tid >> 3) + 64 * i, chunk = tid & 7;
      const int ga = min(m0 + row, p.M - 1), gb = min(n0 + row, p.N - 1);
      u32x4_t za = {0u, 0u, 0u, 0u}, zb = {0u, 0u, 0u, 0u};
      if (chunk < nch) {
        za = *(const u32x4_t*)(p.Ae + (int64_t)ga * p.ldae + c0 + chunk * 8);
        zb = *(const u32x4_t*)(p.Be + (int64_t)gb * p.ldbe + c0 + chunk * 8);
      }
      *(u32x4_t*)&sa[swz(row, chunk)] = za;
      *(u32x4_t*)&sb[swz(row, chunk)] = zb;
    }
    __syncthreads();
    compute(smem, (nch * 8 + 15) >> 4);
    __syncthreads();
  }

  // ---- epilogue ----
  // acc[mt][nt][v] holds C[row][col] with
  //   row = wm*128 + mt*32 + 8*(v/4) + 4*(lane/32) + v%4,  col = wn*64 + nt*32 + lane%32.
  // Each 32-row slab (one mt) of a wave's 128 x 64 tile goes through LDS
  // (fp32, padded pitch) so that the global side moves 16 contiguous bytes
  // per lane; register indices stay compile-time constants.
  constexpr int SP = 72;  // floats per staged row: 4*SP = 32 mod 64 banks
  float* stage = reinterpret_cast<float*>(smem) + wave * (32 * SP);  // fits in the ring
  const int row0 = m0 + wm * 128;
  const int col0 = n0 + wn * 64;
  // the activation is fixed per launch: one branch here, none per value
  auto slabs = [&](auto act_c) {
    constexpr int ACT = decltype(act_c)::value;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      // ACT_BWD: this slab's g and u are fetched before the staging so that
      // their latency overlaps it (rows past M read nothing)
      u32x4_t gw[4], uw[4];
      if (EPI == EPI_ACT_BWD) {
        const int cc = (lane & 7) * 8;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = row0 + mt * 32 + q * 8 + (lane >> 3), col = col0 + cc;
          gw[q] = u32x4_t{0u, 0u, 0u, 0u};
          uw[q] = u32x4_t{0u, 0u, 0u, 0u};
          if (row < p.M && col < p.N) {
            const int64_t o = (int64_t)row * p.hdim + col;
            gw[q] = *(const u32x4_t*)(p.g_in + o);
            uw[q] = *(const u32x4_t*)(p.u_in + o);
          }
        }
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          stage[(8 * (v >> 2) + 4 * (lane >> 5) + (v & 3)) * SP + nt * 32 + (lane & 31)] = acc[mt][nt][v];
      wave_sync();   // the staging region is this wave's own
      if (EPI == EPI_STORE) {
        // lane: 8 consecutive columns of one row per step, 8 rows per step
        const int cc = (lane & 7) * 8;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int rr = q * 8 + (lane >> 3);
          const int row = row0 + mt * 32 + rr;
          const int col = col0 + cc;
          const f32x4_t x0 = *(const f32x4_t*)&stage[rr * SP + cc];
          const f32x4_t x1 = *(const f32x4_t*)&stage[rr * SP + cc + 4];
          if (row < p.M && col < p.N) {
            u32x4_t o;
            o[0] = pack_bf16x2(x0[0], x0[1]);
            o[1] = pack_bf16x2(x0[2], x0[3]);
            o[2] = pack_bf16x2(x1[0], x1[1]);
            o[3] = pack_bf16x2(x1[2], x1[3]);
            *(u32x4_t*)(p.C + (int64_t)row * p.ldc + col) = o;
          }
        }
      } else if (EPI == EPI_GATEUP) {
        // staged columns: [gate j0..j0+31 | up j0..j0+31], j0 = col0 / 2
        const int jj = (lane & 3) * 8;
        const int64_t j = (int64_t)(col0 >> 1) + jj;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int rr = q * 16 + (lane >> 2);
          const int row = row0 + mt * 32 + rr;
          const float* gs = &stage[rr * SP + jj];
          const float* us = gs + 32;
          if (row < p.M && col0 < p.N) {
            float gv[8], uv[8];
            *(f32x4_t*)gv = *(const f32x4_t*)gs;
            *(f32x4_t*)(gv + 4) = *(const f32x4_t*)(gs + 4);
            *(f32x4_t*)uv = *(const f32x4_t*)us;
            *(f32x4_t*)(uv + 4) = *(const f32x4_t*)(us + 4);
            u32x4_t og, ou, oh;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float hv[2];
              uint32_t gb[2], ub[2];
#pragma unroll
              for (int t = 0; t < 2; ++t) {
                gb[t] = f32_to_bf16(gv[2 * e + t]);
                ub[t] = f32_to_bf16(uv[2 * e + t]);
                hv[t] = act_fwd_t<ACT>(bf16_to_f32(gb[t])) * bf16_to_f32(ub[t]);
              }
              og[e] = gb[0] | (gb[1] << 16);
              ou[e] = ub[0] | (ub[1] << 16);
              oh[e] = pack_bf16x2(hv[0], hv[1]);
            }
            const int64_t o = (int64_t)row * p.hdim + j;
            *(u32x4_t*)(p.g_out + o) = og;
            *(u32x4_t*)(p.u_out + o) = ou;
            *(u32x4_t*)(p.h_out + o) = oh;
          }
        }
      } else {  // EPI_ACT_BWD: staged values are dH
        const int cc = (lane & 7) * 8;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int rr = q * 8 + (lane >> 3);
          const int row = row0 + mt * 32 + rr;
          const int col = col0 + cc;
          if (row < p.M && col < p.N) {
            float dh[8];
            *(f32x4_t*)dh = *(const f32x4_t*)&stage[rr * SP + cc];
            *(f32x4_t*)(dh + 4) = *(const f32x4_t*)&stage[rr * SP + cc + 4];
            u32x4_t odg, odu;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float dg[2], du[2];
#pragma unroll
              for (int t = 0; t < 2; ++t) {
                const float g = bf16_to_f32(t ? (gw[q][e] >> 16) : (gw[q][e] & 0xFFFFu));
                const float u = bf16_to_f32(t ? (uw[q][e] >> 16) : (uw[q][e] & 0xFFFFu));
                float a, da;
                act_fwd_bwd_t<ACT>(g, &a, &da);
                const float d = dh[2 * e + t];
                dg[t] = d * u * da;
                du[t] = d * a;
              }
              odg[e] = pack_bf16x2(dg[0], dg[1]);
              odu[e] = pack_bf16x2(du[0], du[1]);
            }
            const int64_t od = (int64_t)row * (2 * p.hdim) + col;
            *(u32x4_t*)(p.dgu + od) = odg;
            *(u32x4_t*)(p.dgu + od + p.hdim) = odu;
          }
        }
      }
      wave_sync();
    }
  };
  if ((EPI == EPI_GATEUP || EPI == EPI_ACT_BWD) && p.act != 0)
    slabs(std::integral_constant<int, 1>());
  else
    slabs(std::integral_constant<int, 0>());
}


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
}  // namespace

template <int EPI, bool SEGA>
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
  auto load_frag_at = [&](Frag& f, const uint8_t* sa, const uint8_t* sb, int ks) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) f.a[mt] = *(const bf16x8_t*)(sa + fq + mt * 256 + fpos(ks));
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) f.b[nt] = *(const bf16x8_t*)(sb + gq + nt * 256 + fpos(ks));
  };
  auto load_frag = [&](Frag& f, int st, int ks) { load_frag_at(f, slot(2 * st), slot(2 * st + 1), ks); };
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

  // ---- main loop ----
  // Step s frees the slots of step s-1, so it issues H_2s+3 (B of step s+1,
  // for s >= 1: the prologue has B of step 1) over its first two substeps and
  // H_2s+4 (A of step s+2) over its second and third, then waits for step
  // s+1's A and B; A of step s+2, issued last, may stay in flight (vmcnt
  // retires in order).
  const int ns = kt1 - kt0, nh = 2 * ns;
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
  using T_ = std::integral_constant<bool, true>;
  using F_ = std::integral_constant<bool, false>;
  if (ns >= 3) {
    step(0, F_(), T_());
    for (int st = 1; st < ns - 2; ++st) step(st, T_(), T_());
    step(ns - 2, T_(), F_());
    step(ns - 1, F_(), F_());
  } else {
    for (int st = 0; st < ns; ++st) step(st, F_(), F_());
  }
  // GATEUP row product: the rank-r fragments of the wave's 64 H columns,
  // loaded here so that the wait below covers them. Waited for later, behind
  // the epilogue's conditional stores, they would cost a wait for all of those.
  const bool rp_on = (EPI == EPI_GATEUP || EPI == EPI_ACT_BWD) && p.rp_r > 0;
  bf16x8_t rpb[2];
  if (EPI == EPI_GATEUP && rp_on) {
    const int jr = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const int64_t c = (int64_t)((n0 + wn * 128) >> 1) + 32 * kc + 8 * kq;
      rpb[kc] = bf16x8_t{};
      if (jr < p.rp_r && c < p.hdim) rpb[kc] = *(const bf16x8_t*)(p.rp_l + (int64_t)jr * p.rp_ldl + c);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  wait_vm<0>();
  __syncthreads();

  // ACT_BWD row product: the rank-r operand over the tile's 256 columns
  // (gate rows 0-15, then up rows 16-31: 32 x 256 bf16) is brought by DMA
  // into the end of the last ring slot, which nothing else uses from here on;
  // the wait of the K-extension (or the one before the epilogue) covers it,
  // so the epilogue reads it from LDS. Row i keeps logical 16-byte chunk c at
  // physical chunk c ^ (i & 15) of its 512 bytes: the 16 rows of a fragment
  // read hit 16 different bank groups. Rows j >= rp_r and columns at or past
  // hdim load as zeros.
  constexpr int RPL_OFF = 5 * G_SLOT - 16384;
  if (EPI == EPI_ACT_BWD && rp_on) {
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
  }

  // ---- K-extension (LoRA up-projection): 64-wide steps over Ae / Be in
  // slots 0 and 1, same layout; columns at or past KE read as zeros; split 0
  // only ----
  if (p.KE > 0 && ksp == 0) {
    const uint64_t eA = (uint64_t)(p.Ae + (int64_t)m0 * p.ldae), eB = (uint64_t)(p.Be + (int64_t)n0 * p.ldbe);
    const int neA = rec_bytes(rowsA, p.ldae);
    const int neB = rec_bytes(rowsB, p.ldbe);
    for (int e = 0; e * BK < p.KE; ++e) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = drow(j), c = e * BK + dcol(j);   // c < KE covers all 8 columns (KE % 16 == 0)
        const bool in = c < p.KE;
        bload_lds<16>(eA, neA, slot(0) + (8 * wave + j) * 1024, in ? (uint32_t)(row * p.ldae + c) * 2u : OOB, 0);
        bload_lds<16>(eB, neB, slot(1) + (8 * wave + j) * 1024, in ? (uint32_t)(row * p.ldbe + c) * 2u : OOB, 0);
      }
      wait_vm<0>();
      ring_barrier();
      const int nsub = (min(BK, p.KE - e * BK) + 15) >> 4;
      for (int ks = 0; ks < nsub; ++ks) {
        Frag f;
        load_frag_at(f, slot(0), slot(1), ks);
        mma(f);
      }
      __syncthreads();
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
  auto slab = [&](auto mt_c, auto act_c) {
    constexpr int mt = decltype(mt_c)::value;
    constexpr int ACT = decltype(act_c)::value;
    auto grow = [&](int s) { return m0 + wm * 128 + 8 * (s >> 1) + 2 * mt + (s & 1); };
    // ACT_BWD: fetch this slab's g and u first so that their latency overlaps
    // the staging (rows past M read nothing)
    u32x4_t gw[8], uw[8];
    if (EPI == EPI_ACT_BWD) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        // staged row q * 4 + lane / 16 is tile row grow(lane / 16) + 16 q
        const int row = grow(lane >> 4) + 16 * q, col = col0 + (lane & 15) * 8;
        gw[q] = u32x4_t{0u, 0u, 0u, 0u};
        uw[q] = u32x4_t{0u, 0u, 0u, 0u};
        if (row < p.M && col < p.N) {
          const int64_t o = (int64_t)grow(lane >> 4) * p.hdim + col + (int64_t)(16 * q) * p.hdim;
          gw[q] = *(const u32x4_t*)(p.g_in + o);
          uw[q] = *(const u32x4_t*)(p.u_in + o);
        }
      }
    }
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
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int s = q * 4 + (lane >> 4);
        const int row = row0 + 16 * q;
        u32x4_t odg = u32x4_t{0u, 0u, 0u, 0u}, odu = u32x4_t{0u, 0u, 0u, 0u};
        if (row < p.M && col < p.N) {
          const float* x = &stage[s * SP + cc];
          if ((EPI == EPI_STORE || EPI == EPI_STORE3) && nsplit > 1) {   // fp32 partial
            float* o = p.part + poff0 + (int64_t)(16 * q) * p.N;
            const f32x4_t x0 = *(const f32x4_t*)x, x1 = *(const f32x4_t*)(x + 4);
            *(f32x4_t*)o = f32x4_t{x0[0], x1[0], x0[1], x1[1]};
            *(f32x4_t*)(o + 4) = f32x4_t{x0[2], x1[2], x0[3], x1[3]};
          } else if (EPI == EPI_STORE || EPI == EPI_STORE3) {
            const f32x4_t x0 = *(const f32x4_t*)x, x1 = *(const f32x4_t*)(x + 4);
            u32x4_t o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(x0[e], x1[e]);
            *(u32x4_t*)(cbase + coff0 + (int64_t)(16 * q) * cld) = o;
          } else {  // staged values are dH
            const f32x4_t x0 = *(const f32x4_t*)x, x1 = *(const f32x4_t*)(x + 4);
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
      }
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
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int s = q * 8 + (lane >> 3);
        const int row = row0 + 32 * q;
        u32x4_t oh = u32x4_t{0u, 0u, 0u, 0u};
        if (row < p.M && col0 < p.N) {
          const float* gs = &stage[s * SP + gcol];
          const float* us = gs + 32;
          const f32x4_t g0 = *(const f32x4_t*)gs, g1 = *(const f32x4_t*)(gs + 4);
          const f32x4_t u0 = *(const f32x4_t*)us, u1 = *(const f32x4_t*)(us + 4);
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
  auto slabs = [&](auto act_c) {
    slab(std::integral_constant<int, 0>(), act_c);
    slab(std::integral_constant<int, 1>(), act_c);
    slab(std::integral_constant<int, 2>(), act_c);
    slab(std::integral_constant<int, 3>(), act_c);
  };
  if ((EPI == EPI_GATEUP || EPI == EPI_ACT_BWD) && p.act != 0)
    slabs(std::integral_constant<int, 1>());
  else
    slabs(std::integral_constant<int, 0>());
  if (rp_on) {
    // every wave's parked results are in LDS (lgkmcnt(0)); the global stores
    // in flight are not waited for
    wait_vm<63>();
    ring_barrier();
    rowprod_store();
  }
}

template <int BSRC, int EPI>
static hipError_t launch_t(const GemmArgs& a, hipStream_t stream) {
  const int ntm = (a.M + BM - 1) / BM, ntn = (a.N + BN - 1) / BN;
  gemm_nt_kernel<BSRC, EPI><<<dim3(ntm * ntn), dim3(NTHR), 0, stream>>>(a);
  return hipGetLastError();
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

template <int EPI, bool SEGA>
static hipError_t launch_bf16(const GemmArgs& a, hipStream_t stream) {
  const int ntm = (a.M + BM - 1) / BM, ntn = (a.N + BN - 1) / BN;
  const int nsplit = a.splits > 1 ? a.splits : 1;
  if (nsplit > 1) {
    const int nk = a.K / BK, kper = (nk + nsplit - 1) / nsplit;
    if ((EPI != EPI_STORE && EPI != EPI_STORE3) || !a.part || a.N % 8 || (nsplit - 1) * kper >= nk)
      return hipErrorInvalidValue;
  }
  gemm_bf16_kernel<EPI, SEGA><<<dim3(ntm * ntn * nsplit), dim3(256), 0, stream>>>(a);
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
  if (a.A1 || a.splits > 1) return hipErrorInvalidValue;
  switch (a.epi) {
    case EPI_STORE: return launch_t<BSRC, EPI_STORE>(a, stream);
    case EPI_GATEUP: return launch_t<BSRC, EPI_GATEUP>(a, stream);
    case EPI_ACT_BWD: return launch_t<BSRC, EPI_ACT_BWD>(a, stream);
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
