// a6: grouped GEMM running the SwiGLU expert FFN over ragged groups.
//
// "Moe dynamic redundancy" (code review, rerouting comment) runs the local
// experts as one grouped matmul over their group sizes, redundant slots
// included; a replica slot computes with its home expert's weights.  The
// FFN itself is SwiGLU: act = SiLU(x Wg^T) * (x Wu^T), out = act Wd^T.
//
// bf16 path: two launches per pass.
//  * GEMM1 (A rows against Wg and Wu [F,H]): a tile computes 128 act columns
//    as 128 gate + 128 up columns held side by side in one 256-row weight
//    tile, so the SwiGLU epilogue finds the gate and up value of an element
//    in the same lane and register.  A rows are gathered through the pass's
//    row index (from x, or from the dedup buffer), so the layer never
//    writes a permuted copy of x.
//  * GEMM2 (act [N,F] against Wd [H,F]): a BM x 256 output tile.
// Both use v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  512 threads =
// 8 waves, in a 4 x 2 grid (256-row tiles: 64 x 128 per wave) or a 2 x 4
// grid (128-row tiles: 64 x 64 per wave) of 32 x 32 MFMA tiles.
//
// Operands go from HBM straight into LDS (buffer_load ... lds, 16 bytes per
// lane, no staging registers) through a ring of NST stages of BK columns,
// so NST-1 stages of loads are in flight while one is multiplied.  Shapes:
// BM=256, BK=64, 2 stages (128 KB LDS) for long reductions (H >= 2048),
// where the taller tile halves the operand traffic per flop; otherwise
// BM=128, BK=32, 3 stages (72 KB), so two workgroups share a CU and one's
// tile set-up, first loads and epilogue overlap the other's MFMAs.  A
// 256-row kernel runs a group's short last tile as BM=128, BK=64, 3 stages.
// In LDS the 16-byte chunks of each row are XOR-permuted by row, so the
// fragment reads of consecutive rows at one chunk hit distinct banks.  Rows
// of A past the group read as zero (an offset past the buffer's byte range)
// and their results are not stored.
//
// Tiles: every group owns ceil(rows/BM) m-tiles (an exclusive scan over
// groups, with an m-tile -> group map, computed with the layout), so empty
// groups cost nothing.  With BM = 256, a group's last m-tile runs as a
// 128-row tile when it holds at most 128 rows.  Tiles are ordered in bands
// of up to GM m-tiles, n-tile by n-tile.  Workgroups are dispatched
// round-robin over the 8 XCDs; each round of as many blocks as the chip
// holds at once covers a run of that order and each XCD a contiguous eighth
// of the run, so the blocks an XCD runs together cover a few m-tiles by a
// few n-tiles of one expert and share both operand panels in its L2, and
// every XCD gets the same share of tall and short tiles.
#include <atomic>
#include <mutex>
#include <type_traits>

#include "common.h"

namespace moe {

namespace {

constexpr int BNB = 256;  // weight rows per tile
typedef int v4i __attribute__((ext_vector_type(4)));
#ifndef MOE_GEMM_GM
#define MOE_GEMM_GM 8
#endif
constexpr int GM = MOE_GEMM_GM;  // m-tiles per band of the tile order
// Bands of the tile order aligned to groups (1) or cut through the whole
// run of m-tiles (0).
#ifndef MOE_GEMM_GBAND
#define MOE_GEMM_GBAND 1
#endif

// Tile shapes <BM, BK, stages, waves, waves along N>: BIG for long
// reductions, SMALL for the rest, and REM, the 128-row shape a BIG kernel
// runs for a group's last tile of at most 128 rows (same wave count as BIG).
// REM uses a 2 x 4 wave grid (64 x 64 per wave): 4 fragment reads per 4
// MFMAs instead of 5 with 4 x 2.
#ifndef MOE_GEMM_BIG
#define MOE_GEMM_BIG 256, 64, 2, 8, 2
#endif
#ifndef MOE_GEMM_SMALL
#define MOE_GEMM_SMALL 128, 32, 3, 8, 4
#endif
#ifndef MOE_GEMM_REM
#define MOE_GEMM_REM 128, 64, 3, 8, 4
#endif
// Tile shapes whose passes run GEMM1 and GEMM2 as one launch (bit 0: 128-row
// tiles, bit 1: 256-row tiles); the others run two launches.  Measured on
// MI355X: one launch is 5% faster on the mid-sized layer (128-row tiles) and
// 10-20% slower on the 256-row shapes, whose two-launch tile order keeps
// every XCD on the same few experts at a time.
#ifndef MOE_GEMM_FUSE
#define MOE_GEMM_FUSE 1
#endif
constexpr int shape_rows(int bm, int, int, int, int) { return bm; }
constexpr int shape_waves(int, int, int, int nw, int) { return nw; }
constexpr int shape_ring(int bm, int bk, int nst, int, int) { return nst * (bm + BNB) * bk * 2; }
constexpr int kRemBM = shape_rows(MOE_GEMM_REM);
constexpr int kRemRing = shape_ring(MOE_GEMM_REM);
constexpr int kPpRing = 10 * 128 * 128;  // the 256-row loop's ten 16 KB quarters

struct GemmParams {
  const uint16_t* A;       // row source (whole array; rows past a group read as zero)
  const int* a_index;      // row n of the pass = A row a_index[n] / a_div, or n when null
  long long a_index_stride;
  int a_div, a_rows;       // a_rows: rows of A (its byte range)
  const uint16_t* B0;      // gate weights (GEMM1) or down weights (GEMM2)
  const uint16_t* B1;      // up weights (GEMM1)
  size_t b_stride;         // elements per expert
  uint16_t* C;
  const int* group_offsets;
  const int* tile_off;
  const int* tile_group;
  int go_stride, tg_stride;  // per layout j
  const int* slot_expert;
  int G, K, Nout, lo_slot, e_base, e_res, n_ntiles;
  int round_blocks;        // blocks per round of the tile order (a multiple of 8):
                           // the blocks resident on the chip at once
  int mt_cap;              // fused kernel: m-tiles its completion flags can hold
  long long max_rows;
  PassArgs pa;
  int* err;                // MOE_ERR_* bits are OR-ed in here (may be null)
  int spin_limit;          // fused kernel: sleeps before a wait gives up (< 0: at once)
  // GEMM1 as the backward's recompute (two-launch kernel only): with d_h
  // set, the epilogue reads d_a [rows, Nout] and writes the SwiGLU backward,
  // d_h [rows, 2 Nout] = (d_hg | d_hu), with the activation in C
  const uint16_t* d_a = nullptr;
  uint16_t* d_h = nullptr;
  // reduction-major B (the 256-row loop's BKM mode): B0 [e_res][k_split][Nout]
  // holds rows k < k_split, B1 [e_res][K - k_split][Nout] the rest
  int k_split = 0;
  // the recompute with ungated d_a (the layer backward): d_a holds u = dy Wd
  // for each row, the row's gate is row_gate[r]; the SwiGLU backward takes
  // d_a = gate * u, C receives gate * act, and dg_part[r * (Nout / 32) + b]
  // the sum over act columns 32 b .. 32 b + 31 of u * act (the row's gate
  // gradient in parts)
  const float* row_gate = nullptr;
  float* dg_part = nullptr;
};

// The SwiGLU backward of one output element from the gate and up
// pre-activations and d_a: act = SiLU(g) u, d_hg = d_a u SiLU'(g), d_hu =
// d_a SiLU(g), SiLU'(g) = s (1 + g (1 - s)) with s the logistic of g (the
// forward's SiLU, hardware reciprocal).
// With the row's gate rg (1 when d_a is already gated) d_a = rg * (stored
// d_a) and C receives rg * act; returns (stored d_a) * act, act as stored in
// bf16, the element's term of the row's gate gradient.
__device__ __forceinline__ float swiglu_bwd_store(const GemmParams& P, size_t r, int c, float gv,
                                                  float uv, float rg) {
  const float u = bf2f(P.d_a[r * P.Nout + c]);
  const float da = u * rg;
  const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-gv));
  const float silu = gv * sg;
  const float act = silu * uv;
  P.C[r * P.Nout + c] = f2bf(act * rg);
  P.d_h[r * 2 * P.Nout + c] = f2bf(da * uv * (sg * (1.0f + gv * (1.0f - sg))));
  P.d_h[r * 2 * P.Nout + P.Nout + c] = f2bf(da * silu);
  return u * bf2f(f2bf(act));
}

// Reports an error bit found by the device (one report per block).
__device__ __forceinline__ void report(int* err, int bit) {
  if (err != nullptr && threadIdx.x == 0) atomicOr(err, bit);
}

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  // raw buffer: loads at offsets >= bytes return zero
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Chunk permutation of LDS row `row`: the fragment reads of consecutive
// rows at one logical chunk land on distinct banks (both permutations were
// measured free of LDS bank conflicts on gfx950 with SQ_LDS_BANK_CONFLICT).
template <int BK>
__device__ __forceinline__ int swz(int row) {
  if (BK == 64) return ((row >> 1) ^ ((row & 1) << 2)) & 7;
  return (row >> 2) & 3;
}

// Waits until at most N of this wave's global->LDS loads are outstanding
// and all of its LDS reads have returned, then joins the workgroup barrier:
// after it, every wave's loads of the awaited stage have landed and no wave
// still reads the buffer the next loads overwrite.  The memory clobber keeps
// the compiler from moving LDS accesses across it.
template <int N>
__device__ __forceinline__ void vm_wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Waits until at most N of this wave's global->LDS loads are outstanding
// (no barrier).
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void lgkm_wait0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Workgroup barrier that no instruction is scheduled across (the phases of
// the two wave groups must not bleed into each other).
__device__ __forceinline__ void pp_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16 as inline asm (the builtin would make the compiler
// wait for the ring's in-flight LDS-direct loads first): within each
// 16-lane group, output lane 4a+b receives element b of the 8-byte runs
// that lanes a, a+4, a+8 and a+12 address.  Pending until tie_wait.
template <int OFF>
__device__ __forceinline__ void lds_read_tr(v4i16& r, unsigned addr) {
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
}

// Waits for every LDS read of the wave; the 16 registers are tied to the
// wait so that no use of them is placed before it.
__device__ __forceinline__ void tie_wait(v4i16 (&r)[16]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]),
                 "+v"(r[6]), "+v"(r[7]), "+v"(r[8]), "+v"(r[9]), "+v"(r[10]), "+v"(r[11]),
                 "+v"(r[12]), "+v"(r[13]), "+v"(r[14]), "+v"(r[15]));
}

__device__ __forceinline__ bf16x8 join_halves(const v4i16& lo, const v4i16& hi) {
  bf16x8 v;
  __builtin_memcpy(&v, &lo, 8);
  __builtin_memcpy(reinterpret_cast<char*>(&v) + 8, &hi, 8);
  return v;
}

// 16-byte chunk permutation of a 256-byte LDS row of a reduction-major B
// quarter.  A transpose read takes 32 bytes from each of 16 rows, 8g + k
// (k < 4) for its 16-lane groups g; rows 256 bytes apart share their banks
// (64 banks of 4 bytes).  Row bits 0-1 move the 4 rows of a group to
// disjoint 64-byte windows, and row bit 3 (g odd) to the other 32-byte half
// of each window, so the 512 bytes of a read cover every bank exactly twice
// (with bits 0-1 alone, groups 0-3 shared 32 banks: twice the cycles).
__device__ __forceinline__ int kswz(int row) { return ((row & 3) << 2) | ((row >> 2) & 2); }

// Starts the loads of K step `step` into its ring stage: each wave-wide
// load fills RPI consecutive rows (1 KB) of the stage.
template <int BM, int BK, int NST, bool SWIGLU, int NW>
__device__ __forceinline__ void gmm_issue(char* smem, int step, int w,
                                          __amdgpu_buffer_rsrc_t ra_r, __amdgpu_buffer_rsrc_t rb0,
                                          __amdgpu_buffer_rsrc_t rb1,
                                          const int* a_off, const int* b_off) {
  constexpr int RB = BK * 2, RPI = 1024 / RB;
  constexpr int AI = BM / RPI / NW, BI = BNB / RPI / NW;
  constexpr int SA = BM * RB, SS = (BM + BNB) * RB;
  char* st = smem + (step % NST) * SS;
  const int kb = step * BK * 2;
#pragma unroll
  for (int i = 0; i < AI; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra_r, (lds_void*)(st + (i * NW + w) * RPI * RB), 16,
                                             a_off[i], kb, 0, 0);
#pragma unroll
  for (int i = 0; i < BI; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(SWIGLU && i >= BI / 2 ? rb1 : rb0,
                                             (lds_void*)(st + SA + (i * NW + w) * RPI * RB), 16,
                                             b_off[i], kb, 0, 0);
}

// Reads the A and B fragments of K slice ks (16 columns) of one stage, for
// the wave's first LV 32-row MFMA tiles (the rest hold only rows past the
// group).
template <int BK, int MI, int NI, int LV>
__device__ __forceinline__ void gmm_frags(const char* sa, const char* sb, const int (&a_row)[MI],
                                          const int (&b_row)[NI], int lane, int ks,
                                          bf16x8 (&a)[MI], bf16x8 (&b)[NI]) {
  if (LV == 0) return;
  constexpr int RB = BK * 2;
  const int kc = ks * 2 + (lane >> 5);
#pragma unroll
  for (int mi = 0; mi < LV; ++mi)
    a[mi] = *(const bf16x8*)(sa + a_row[mi] * RB + ((kc ^ swz<BK>(a_row[mi])) << 4));
#pragma unroll
  for (int ni = 0; ni < NI; ++ni)
    b[ni] = *(const bf16x8*)(sb + b_row[ni] * RB + ((kc ^ swz<BK>(b_row[ni])) << 4));
}

template <int MI, int NI, int LV>
__device__ __forceinline__ void gmm_mma(const bf16x8 (&a)[MI], const bf16x8 (&b)[NI],
                                        floatx16 (&acc)[MI][NI]) {
#pragma unroll
  for (int mi = 0; mi < LV; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
      acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
}

// Calls f(std::integral_constant<int, min(live, L)>) for live >= 0.
template <int L, class F>
__device__ __forceinline__ void live_dispatch(int live, F& f) {
  if constexpr (L == 0) {
    f(std::integral_constant<int, 0>{});
  } else {
    if (live >= L) f(std::integral_constant<int, L>{});
    else live_dispatch<L - 1>(live, f);
  }
}

// One BM x 256 tile (GEMM1: BM x 128 act columns) of group rows
// [row0, row0 + rows), rows <= BM, of weight n-tile nt of local expert e;
// smem holds at least NST * (BM + 256) * BK * 2 bytes.  COH (GEMM1 of the
// one-launch kernel only): the act rows are stored with cache policy sc1,
// written through the XCD's L2 to the memory side that every XCD reads, so
// a GEMM2 tile of the same launch on another XCD can read them.  The GEMM2
// side loads with the default policy; what makes that safe is stated at
// the one-launch kernel.
template <int BM, int BK, int NST, int NW, int NWN, bool SWIGLU, bool COH = false>
__device__ __forceinline__ void gmm_tile(const GemmParams& P, char* smem, const int* aidx,
                                         int row0, int rows, int nt, int e) {
  constexpr int RB = BK * 2;          // LDS bytes per row of a stage
  constexpr int CPR = BK / 8;         // 16-byte chunks per row
  constexpr int RPI = 1024 / RB;      // rows one wave-wide load fills
  constexpr int AI = BM / RPI / NW;   // A loads per wave per stage
  constexpr int BI = BNB / RPI / NW;  // B loads per wave per stage
  constexpr int LPS = AI + BI;
  constexpr int SA = BM * RB, SS = (BM + BNB) * RB;
  constexpr int WM = BM / (NW / NWN);  // rows per wave (waves form (NW/NWN) x NWN)
  constexpr int MI = WM / 32;          // 32-row MFMA tiles per wave
  constexpr int NI = BNB / NWN / 32;   // 32-column MFMA tiles per wave
  static_assert(NI >= 2 && NI % 2 == 0, "a SwiGLU wave pairs gate and up tiles");
  static_assert(AI >= 1 && BI >= 2 && MI >= 1, "tile shape");
  static_assert(NST >= 2 && NST <= 5, "stages");


  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w / NWN, wn = w % NWN;
  const int K = P.K;
  const int KT = K / BK;

  // A as one raw buffer over its whole source; each lane's rows come from
  // the row index (gathered rows) or are the pass rows themselves.  Rows
  // past the group get an offset beyond the buffer and read as zero.
  const __amdgpu_buffer_rsrc_t ra_r = make_rsrc(P.A, (unsigned)P.a_rows * K * 2);
  __amdgpu_buffer_rsrc_t rb0, rb1;
  if (SWIGLU) {
    rb0 = make_rsrc(P.B0 + (size_t)e * P.b_stride + (size_t)nt * 128 * K, 128u * K * 2);
    rb1 = make_rsrc(P.B1 + (size_t)e * P.b_stride + (size_t)nt * 128 * K, 128u * K * 2);
  } else {
    rb0 = make_rsrc(P.B0 + (size_t)e * P.b_stride + (size_t)nt * 256 * K, 256u * K * 2);
    rb1 = rb0;
  }
  // global byte offsets of this lane's chunk in each of its loads
  int a_off[AI], b_off[BI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    int row = (i * NW + w) * RPI + lane / CPR;
    int src = -1;
    if (row < rows) src = aidx ? aidx[row0 + row] / P.a_div : row0 + row;
    a_off[i] = (src >= 0 && src < P.a_rows)
                   ? src * K * 2 + (((lane % CPR) ^ swz<BK>(row)) << 4)
                   : (int)0x80000000;
  }
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    int row = (i * NW + w) * RPI + lane / CPR;
    int wr = SWIGLU ? (row & 127) : row;
    b_off[i] = wr * K * 2 + (((lane % CPR) ^ swz<BK>(row)) << 4);
  }

  // fragment read offsets (bytes within a stage) for chunk kc of each row
  int a_row[MI], b_row[NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) a_row[mi] = wm * WM + mi * 32 + (lane & 31);
#pragma unroll
  // SwiGLU: the wave's gate tiles are its first NI/2, the up tiles of the
  // same act columns its last NI/2 (weight rows 128 + the gate rows)
  for (int ni = 0; ni < NI; ++ni)
    b_row[ni] = (SWIGLU ? ((ni / (NI / 2)) * 128 + wn * (128 / NWN) + (ni % (NI / 2)) * 32)
                        : (wn * (BNB / NWN) + ni * 32)) +
                (lane & 31);

  floatx16 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[mi][ni][q] = 0.0f;

#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (s < KT) gmm_issue<BM, BK, NST, SWIGLU, NW>(smem, s, w, ra_r, rb0, rb1, a_off, b_off);

  // Software pipeline across K steps: the last slice's fragments are read
  // before the barrier, and its MFMAs are issued after it, overlapping the
  // first fragment reads of the next stage.  A wave multiplies only its
  // 32-row MFMA tiles that hold rows of the group (LV of them); padding rows
  // cost it no fragment reads and no MFMAs, so on a short tile the other
  // wave of each SIMD has the matrix pipe to itself.  Every wave still
  // issues its share of the loads and joins every barrier.
  constexpr int NS = BK / 16;  // K slices per step
  static_assert(NS % 2 == 0, "the pending last slice lives in fragment set 1");
  bf16x8 a[2][MI], b[2][NI];
  auto kloop = [&](auto live_c) {
    constexpr int LV = decltype(live_c)::value;
    for (int kt = 0; kt < KT; ++kt) {
      const int ahead = min(KT - 1 - kt, NST - 2);  // stages allowed to stay in flight
      if (ahead >= 3) vm_wait_barrier<3 * LPS>();
      else if (ahead == 2) vm_wait_barrier<2 * LPS>();
      else if (ahead == 1) vm_wait_barrier<LPS>();
      else vm_wait_barrier<0>();
      if (kt + NST - 1 < KT)
        gmm_issue<BM, BK, NST, SWIGLU, NW>(smem, kt + NST - 1, w, ra_r, rb0, rb1, a_off, b_off);
      const char* sa = smem + (kt % NST) * SS;
      const char* sb = sa + SA;
      // slice 0 of this step goes to set 0; slice NS-1 of the previous step
      // is still pending in set 1
      gmm_frags<BK, MI, NI, LV>(sa, sb, a_row, b_row, lane, 0, a[0], b[0]);
      if (kt > 0) gmm_mma<MI, NI, LV>(a[1], b[1], acc);  // last slice of the previous step
#pragma unroll
      for (int ks = 0; ks < NS - 1; ++ks) {
        const int cur = ks & 1;
        gmm_frags<BK, MI, NI, LV>(sa, sb, a_row, b_row, lane, ks + 1, a[cur ^ 1], b[cur ^ 1]);
        gmm_mma<MI, NI, LV>(a[cur], b[cur], acc);
      }
    }
    gmm_mma<MI, NI, LV>(a[(NS - 1) & 1], b[(NS - 1) & 1], acc);
  };
  // 32-row MFMA tiles of this wave that hold rows of the group (wave-uniform)
  const int live = __builtin_amdgcn_readfirstlane(min(MI, max(0, (rows - wm * WM + 31) / 32)));
  live_dispatch<MI>(live, kloop);

  if (SWIGLU && !COH && P.d_h != nullptr) {
    // the backward's recompute: element by element, no LDS (32x32 layout:
    // register q of a lane holds row (q/4)*8 + (lane/32)*4 + q%4, column
    // lane%32; each ni is one 32-column block of the gate-gradient parts)
    const bool gated = P.row_gate != nullptr;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int lr = wm * WM + mi * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
        const bool ok = lr < rows;
        const float rg = gated && ok ? P.row_gate[row0 + lr] : 1.0f;
#pragma unroll
        for (int ni = 0; ni < NI / 2; ++ni) {
          const int c0 = nt * 128 + wn * (128 / NWN) + ni * 32;
          float t = 0.0f;
          if (ok)
            t = swiglu_bwd_store(P, (size_t)(row0 + lr), c0 + (lane & 31), acc[mi][ni][q],
                                 acc[mi][ni + NI / 2][q], rg);
          if (gated) {
            // the 32 lanes of a row (wave-uniform branch: every lane shuffles)
#pragma unroll
            for (int o = 16; o >= 1; o >>= 1) t += __shfl_xor(t, o);
            if (ok && (lane & 31) == 0)
              P.dg_part[(size_t)(row0 + lr) * (P.Nout / 32) + c0 / 32] = t;
          }
        }
      }
    __syncthreads();  // as after the LDS epilogue: every wave is done with the ring
    return;
  }
  // Epilogue through LDS: the ring is free once every wave has read its last
  // stage, so the tile is written there in bf16 and then stored as whole
  // 16-byte row chunks (instead of 2-byte stores scattered over rows).
  constexpr int OUTC = SWIGLU ? 128 : BNB;           // output columns of the tile
  constexpr int ROWB = OUTC * 2;                      // bytes per output row
  constexpr int PAD = BM * (ROWB + 16) <= NST * SS ? 16 : 0;  // keeps row r and r+4 apart
  constexpr int STRIDE = ROWB + PAD;
  static_assert(BM * STRIDE <= NST * SS, "output tile fits the ring");
  __syncthreads();
  // 32x32 accumulator layout: register q of a lane holds row
  // (q/4)*8 + (lane/32)*4 + q%4, column lane%32.
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int lr = wm * WM + mi * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
      uint16_t* orow = (uint16_t*)(smem + lr * STRIDE);
      if (SWIGLU) {
#pragma unroll
        for (int ni = 0; ni < NI / 2; ++ni) {
          const float gv = acc[mi][ni][q], uv = acc[mi][ni + NI / 2][q];
          // SiLU(g) * u with the hardware reciprocal (~1 ulp)
          const float av = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
          orow[wn * (128 / NWN) + ni * 32 + (lane & 31)] = f2bf(av);
        }
      } else {
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          orow[wn * (BNB / NWN) + ni * 32 + (lane & 31)] = f2bf(acc[mi][ni][q]);
      }
    }
  }
  __syncthreads();
  constexpr int CPRO = ROWB / 16;                 // 16-byte chunks per output row
  constexpr int RPIO = (64 * NW) / CPRO;          // rows per pass of the block
  static_assert((64 * NW) % CPRO == 0 && BM % RPIO == 0, "store passes");
  uint16_t* cbase = P.C + (size_t)row0 * P.Nout + (size_t)nt * OUTC;
  if (COH && SWIGLU) {
    // stores past the tile's last row fall outside the buffer range and are dropped
    const __amdgpu_buffer_rsrc_t rc =
        make_rsrc(cbase, (unsigned)(((rows - 1) * P.Nout + OUTC) * 2));
#pragma unroll
    for (int it = 0; it < BM / RPIO; ++it) {
      const int r = it * RPIO + tid / CPRO, ch = tid % CPRO;
      if (r < rows)
        __builtin_amdgcn_raw_buffer_store_b128(*(const v4i*)(smem + r * STRIDE + ch * 16), rc,
                                               (r * P.Nout + ch * 8) * 2, 0, 16 /* sc1 */);
    }
    return;
  }
#pragma unroll
  for (int it = 0; it < BM / RPIO; ++it) {
    const int r = it * RPIO + tid / CPRO, ch = tid % CPRO;
    if (r < rows)
      *(uint4*)(cbase + (size_t)r * P.Nout + ch * 8) = *(const uint4*)(smem + r * STRIDE + ch * 16);
  }
}

// One 256 x 256 tile (GEMM1: 256 x 128 act columns) with more than 128
// rows of the group, for long reductions (H >= 2048).  8 waves in two groups
// of four (one wave of each group per SIMD) take turns: while one group
// multiplies, the other reads its fragments of the next K step from LDS and
// issues global->LDS loads, so every SIMD's matrix pipe is fed by one wave
// while the other moves data.
//
// K steps of 64 columns.  Each step's operands are four 16 KB quarters:
// A rows 0-127 (read by group 0), A rows 128-255 (group 1), B rows 0-127
// and B rows 128-255 (both groups); quarter q = 4*step + part lives in LDS
// slot q % 10 (160 KB).  Phases: group 0 reads step k in phase 2k+1 (MEM)
// and multiplies it in phase 2k+2 (COMP), group 1 one phase later, with a
// barrier between phases.  Group 0 issues quarters 4j+7 and 4j+8 in MEM(j),
// group 1 quarters 4j+9 and 4j+10 in MEM(j), each into a slot whose
// previous quarter both groups have read by then; group 0 waits for its
// loads at the end of its COMP phase, group 1 at the end of its MEM phase,
// so every quarter of step k+1 has landed before the barrier after which it
// is read.  The loads are spread over both groups' MEM phases: a wave
// issuing an LDS-direct load stalls until the texture unit accepts it, so
// loads kept off the multiplying wave keep its MFMAs back to back, and two
// quarters per phase keep the unit busy in both phases.
//
// 16x16x32 MFMAs (each wave 64 x 128: 4 x 8 tiles).  Measured on MI355X
// against 32x32x16: the same work takes more cycles but the chip holds a
// higher clock under its power limit, 3-4% faster on dense shapes.
//
// GEMM1's B tile is 128 gate rows (quarter 2) and the 128 up rows of the
// same act columns (quarter 3); a wave takes 64 act columns: 4 gate tiles
// from quarter 2 and the matching 4 up tiles from quarter 3, so the SwiGLU
// epilogue pairs them in registers.  GEMM2's wave takes 128 output columns
// from one B quarter.  A rows past the group read as zero; a wave whose 64
// rows are all past the group skips its reads and MFMAs.
// BKM: B is stored reduction-major ([e][K][Nout], the backward's weights as
// they are), plain GEMM only.  A B quarter then holds 64 reduction rows of
// the quarter's 128 output columns (256 bytes each, chunks permuted by
// kswz), and the B fragments come from two transpose reads each.
template <bool SWIGLU, bool BKM = false>
__device__ __forceinline__ void gmm_tile_pp(const GemmParams& P, char* smem, const int* aidx,
                                            int row0, int rows, int nt, int e) {
  static_assert(!(SWIGLU && BKM), "reduction-major B for the plain GEMM only");
  constexpr int BK = 64, RB = BK * 2, CPR = BK / 8, RPI = 1024 / RB;  // 8 rows per load
  constexpr int QS = 128 * RB;       // bytes per quarter
  constexpr int LQ = 128 / RPI / 4;  // loads per wave per quarter (4)
  constexpr int NQ_PRO = 8;          // quarters of the first two steps
  constexpr int MI = 4, NI = 8;      // 16x16 tiles per wave
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = w >> 2, wig = w & 3;
  const int wml = wig >> 1, wn = wig & 1;
  const int K = P.K, KT = K / BK, NQ = 4 * KT;

  const __amdgpu_buffer_rsrc_t ra = make_rsrc(P.A, (unsigned)P.a_rows * K * 2);
  __amdgpu_buffer_rsrc_t rb0, rb1;
  if (BKM) {
    rb0 = rb1 = make_rsrc(P.B0, 0);  // per quarter in issue_bk
  } else if (SWIGLU) {
    rb0 = make_rsrc(P.B0 + (size_t)e * P.b_stride + (size_t)nt * 128 * K, 128u * K * 2);
    rb1 = make_rsrc(P.B1 + (size_t)e * P.b_stride + (size_t)nt * 128 * K, 128u * K * 2);
  } else {
    rb0 = make_rsrc(P.B0 + (size_t)e * P.b_stride + (size_t)nt * 256 * K, 128u * K * 2);
    rb1 = make_rsrc(P.B0 + (size_t)e * P.b_stride + (size_t)nt * 256 * K + (size_t)128 * K,
                    128u * K * 2);
  }
  // A: a group only ever loads its own quarter (rows grp*128..); load i of
  // wave wig fills rows (i*4 + wig)*8 + lane/8 of it.  B rows are
  // contiguous: rows 32 apart share the chunk swizzle.
  int a_off[LQ];
#pragma unroll
  for (int i = 0; i < LQ; ++i) {
    const int row = (i * 4 + wig) * RPI + lane / CPR;
    const int trow = grp * 128 + row;
    int src = -1;
    if (trow < rows) src = aidx ? aidx[row0 + trow] / P.a_div : row0 + trow;
    a_off[i] = (src >= 0 && src < P.a_rows) ? src * K * 2 + (((lane % CPR) ^ swz<BK>(row)) << 4)
                                           : (int)0x80000000;
  }
  const int brow0 = wig * RPI + lane / CPR;
  const int b_off0 = brow0 * K * 2 + (((lane % CPR) ^ swz<BK>(brow0)) << 4);
  const int b_step = 4 * RPI * K * 2;
  // quarter q's loads: this group's A quarter, or B rows 0-127 / 128-255
  auto issue_a = [&](int q) {
    if (q >= NQ) return;
    char* st = smem + (q % 10) * QS;
    const int kb = (q >> 2) * BK * 2;
#pragma unroll
    for (int i = 0; i < LQ; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(st + (i * 4 + wig) * RPI * RB), 16,
                                               a_off[i], kb, 0, 0);
  };
  auto issue_b = [&](int q, __amdgpu_buffer_rsrc_t rb) {
    if (q >= NQ) return;
    char* st = smem + (q % 10) * QS;
    const int kb = (q >> 2) * BK * 2;
#pragma unroll
    for (int i = 0; i < LQ; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(st + (i * 4 + wig) * RPI * RB), 16,
                                               b_off0 + i * b_step, kb, 0, 0);
  };
  // BKM: load i of wave wig fills quarter rows 4 (4i + wig) + lane/16, 16
  // chunks of 16 bytes each; the quarter's rows are reduction rows 64 s ..
  // 64 s + 63 of step s, from B0 below k_split and B1 above
  int bk_off[LQ];
#pragma unroll
  for (int i = 0; i < LQ; ++i) {
    const int r = (i * 4 + wig) * 4 + (lane >> 4);
    bk_off[i] = r * P.Nout * 2 + (((lane & 15) ^ kswz(r)) << 4);
  }
  auto issue_bk = [&](int q, int half) {
    if (q >= NQ) return;
    char* st = smem + (q % 10) * QS;
    const int k0 = (q >> 2) * BK;
    const bool lo = k0 < P.k_split;
    // B0's experts are b_stride apart; B1's (K - k_split) x Nout
    const uint16_t* base = (lo ? P.B0 + (size_t)e * P.b_stride
                               : P.B1 + (size_t)e * (size_t)(K - P.k_split) * P.Nout) +
                           (size_t)nt * 256 + half * 128;
    const int kr = lo ? k0 : k0 - P.k_split;
    const int krows = lo ? P.k_split : K - P.k_split;
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc(base, (unsigned)((krows - 1) * P.Nout * 2 + 256));
#pragma unroll
    for (int i = 0; i < LQ; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(st + (i * 4 + wig) * 1024), 16,
                                               bk_off[i], kr * P.Nout * 2, 0, 0);
  };
  // BKM fragment reads: lane j of 16-lane group g addresses row 8g + j/4
  // (+4 for the second read) and columns 4 (j%4) .. of the 16-column tile
  const int tj = lane & 15;
  const unsigned tk_base = (8 * (lane >> 4) + (tj >> 2)) * 256 + (tj & 1) * 8 + (((tj & 3) >> 1) << 4);
  const int tk_sw = ((tj >> 2) << 2) | (((lane >> 4) & 1) << 1);  // kswz of the lane's rows
  // fragment rows within their quarters (16x16x32: lane reads row lane%16)
  int ar[MI], br[NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) ar[mi] = wml * 64 + mi * 16 + (lane & 15);
#pragma unroll
  for (int ni = 0; ni < NI; ++ni)
    br[ni] = (SWIGLU ? wn * 64 + (ni & 3) * 16 : ni * 16) + (lane & 15);
  floatx4 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[mi][ni][q] = 0.0f;
  // a wave with no row of the group skips its fragment reads and MFMAs
  const bool live = grp * 128 + wml * 64 < rows;

  // prologue: steps 0 and 1; group 0 its A quarters and B rows 0-127,
  // group 1 its A quarters and B rows 128-255
  if (grp == 0) {
    issue_a(0);
    if (BKM) issue_bk(2, 0); else issue_b(2, rb0);
    issue_a(4);
    if (BKM) issue_bk(6, 0); else issue_b(6, rb0);
  } else {
    issue_a(1);
    if (BKM) issue_bk(3, 1); else issue_b(3, rb1);
    issue_a(5);
    if (BKM) issue_bk(7, 1); else issue_b(7, rb1);
  }
  vm_wait<0>();
  pp_barrier();
  if (grp == 1) pp_barrier();
  bf16x8 a[2][MI], b[2][BKM ? 1 : NI];
  v4i16 bt[2][BKM ? NI : 1][2];  // BKM: the two 4-row halves of each B fragment
  for (int kt = 0; kt < KT; ++kt) {
    const char* sa = smem + ((4 * kt + grp) % 10) * QS;
    const char* sb0 = smem + ((4 * kt + 2) % 10) * QS;
    const char* sb1 = smem + ((4 * kt + 3) % 10) * QS;
    const char* sbw = SWIGLU ? sb0 : (wn ? sb1 : sb0);
    // MEM phase: this group's two quarters (group 0: B rows 128-255 of
    // step kt+1 and its A quarter of step kt+2; group 1: its A quarter and
    // B rows 0-127 of step kt+2), then the step's fragments
    const int q0 = 4 * kt + 7 + 2 * grp, q1 = q0 + 1;
    if (grp == 0) {
      if (q0 >= NQ_PRO) {
        if (BKM) issue_bk(q0, 1); else issue_b(q0, rb1);
      }
      issue_a(q1);
    } else {
      issue_a(q0);
      if (BKM) issue_bk(q1, 0); else issue_b(q1, rb0);
    }
    if (live) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int kc = ks * 4 + (lane >> 4);
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
          a[ks][mi] = *(const bf16x8*)(sa + ar[mi] * RB + ((kc ^ swz<BK>(ar[mi])) << 4));
        if constexpr (!BKM) {
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) {
            const char* sb = SWIGLU ? (ni < 4 ? sb0 : sb1) : sbw;
            b[ks][ni] = *(const bf16x8*)(sb + br[ni] * RB + ((kc ^ swz<BK>(br[ni])) << 4));
          }
        }
      }
      if constexpr (BKM) {
        // rows 32 ks + 8g .. +7 of column 16 ni + lane%16: two transpose
        // reads of 4 rows each, per slice and n-tile
        const unsigned sbw_a =
            (unsigned)(size_t)(const __attribute__((address_space(3))) char*)sbw + tk_base;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) {
            // chunk 2 ni + (j%4)/2 of the lane's rows, permuted by kswz
            const unsigned ad = sbw_a + ((((2 * ni) ^ tk_sw)) << 4);
            if (ks == 0) {
              lds_read_tr<0>(bt[ks][ni][0], ad);
              lds_read_tr<1024>(bt[ks][ni][1], ad);
            } else {
              lds_read_tr<8192>(bt[ks][ni][0], ad);
              lds_read_tr<9216>(bt[ks][ni][1], ad);
            }
          }
          tie_wait(*reinterpret_cast<v4i16(*)[16]>(&bt[ks][0][0]));
        }
      }
    }
    if (grp == 1) {
      // quarters up to 4kt+6 landed; its two newest may stay in flight
      if (q1 < NQ) vm_wait<2 * LQ>();
      else if (q0 < NQ) vm_wait<LQ>();
      else vm_wait<0>();
    }
    lgkm_wait0();
    pp_barrier();
    // COMP phase
    if (live) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) {
            bf16x8 bv;
            if constexpr (BKM) bv = join_halves(bt[ks][ni][0], bt[ks][ni][1]);
            else bv = b[ks][ni];
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks][mi], bv, acc[mi][ni], 0, 0, 0);
          }
    }
    if (grp == 0) {
      // quarters up to 4kt+7 landed; its newest (4kt+8) may stay in flight
      if (q1 >= NQ_PRO && q1 < NQ) vm_wait<LQ>();
      else vm_wait<0>();
    }
    pp_barrier();
  }
  if (grp == 0) pp_barrier();

  if (SWIGLU && P.d_h != nullptr) {
    // the backward's recompute: element by element, no LDS (16x16 layout:
    // register q of a lane holds row (lane/16)*4 + q, column lane%16)
    // (each pair of ni is one 32-column block of the gate-gradient parts)
    const int wr0 = grp * 128 + wml * 64;
    const bool gated = P.row_gate != nullptr;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int lr = wr0 + mi * 16 + (lane >> 4) * 4 + q;
        const bool ok = lr < rows;
        const float rg = gated && ok ? P.row_gate[row0 + lr] : 1.0f;
        float t[2] = {0.0f, 0.0f};
        if (ok) {
#pragma unroll
          for (int ni = 0; ni < 4; ++ni)
            t[ni >> 1] += swiglu_bwd_store(P, (size_t)(row0 + lr),
                                           nt * 128 + wn * 64 + ni * 16 + (lane & 15),
                                           acc[mi][ni][q], acc[mi][ni + 4][q], rg);
        }
        if (gated) {
          // the 16 lanes of a row (wave-uniform branch: every lane shuffles)
#pragma unroll
          for (int o = 8; o >= 1; o >>= 1) {
            t[0] += __shfl_xor(t[0], o);
            t[1] += __shfl_xor(t[1], o);
          }
          if (ok && (lane & 15) == 0) {
            float* pr = P.dg_part + (size_t)(row0 + lr) * (P.Nout / 32) + (nt * 128 + wn * 64) / 32;
            pr[0] = t[0];
            pr[1] = t[1];
          }
        }
      }
    __syncthreads();
    return;
  }
  // Epilogue through LDS (the ring is free: every wave passed the last
  // barrier after its last reads), then whole 16-byte row chunks.
  // 16x16 accumulator layout: register q of a lane holds row
  // (lane/16)*4 + q, column lane%16.
  constexpr int OUTC = SWIGLU ? 128 : BNB;
  constexpr int ROWB = OUTC * 2;
  constexpr int STRIDE = ROWB + 16;
  static_assert(256 * STRIDE <= 10 * QS, "output tile fits the ring");
  const int wm0 = grp * 128 + wml * 64;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int lr = wm0 + mi * 16 + (lane >> 4) * 4 + q;
      uint16_t* orow = (uint16_t*)(smem + lr * STRIDE);
      if (SWIGLU) {
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const float gv = acc[mi][ni][q], uv = acc[mi][ni + 4][q];
          // SiLU(g) * u with the hardware reciprocal (~1 ulp)
          const float av = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
          orow[wn * 64 + ni * 16 + (lane & 15)] = f2bf(av);
        }
      } else {
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          orow[wn * 128 + ni * 16 + (lane & 15)] = f2bf(acc[mi][ni][q]);
      }
    }
  __syncthreads();
  constexpr int CPRO = ROWB / 16;
  constexpr int RPIO = 512 / CPRO;
  uint16_t* cbase = P.C + (size_t)row0 * P.Nout + (size_t)nt * OUTC;
#pragma unroll
  for (int it = 0; it < 256 / RPIO; ++it) {
    const int r = it * RPIO + tid / CPRO, ch = tid % CPRO;
    if (r < rows)
      *(uint4*)(cbase + (size_t)r * P.Nout + ch * 8) = *(const uint4*)(smem + r * STRIDE + ch * 16);
  }
}

template <int BM, int BK, int NST, bool SWIGLU, int NW, int NWN, bool BKM = false>
__global__ __launch_bounds__(64 * NW, 1) void gmm_bf16_kernel(GemmParams P) {
  // one ring for either tile shape the kernel may run; 256-row tiles run
  // the two-group loop over its 160 KB ring of quarters (with reduction-major
  // B every tile does, short ones too)
  static_assert(!BKM || BM == 256, "reduction-major B in the 256-row loop only");
  constexpr bool HAS_REM = BM > kRemBM && !BKM;
  constexpr int RING = BM == 256 ? kPpRing : NST * (BM + BNB) * BK * 2;
  static_assert(BM != 256 || NW == 8, "the 256-row loop runs 8 waves");
  static_assert(!HAS_REM || shape_waves(MOE_GEMM_REM) == NW, "REM runs in the same block");
  __shared__ __attribute__((aligned(1024))) char smem[HAS_REM && kRemRing > RING ? kRemRing : RING];
  PassInfo pi = resolve_pass(P.pa);
  if (!pi.active) return;
  const int* group_offsets = P.group_offsets + (size_t)pi.j * P.go_stride;
  const int* tile_off = P.tile_off + (size_t)pi.j * P.go_stride;
  const int* tile_group = P.tile_group + (size_t)pi.j * P.tg_stride;
  const int total_mt = tile_off[P.G];
  if (group_offsets[P.G] > P.max_rows || total_mt < 0) {  // malformed: touch nothing
    if (blockIdx.x == 0) report(P.err, MOE_ERR_BAD_OFFSETS);
    return;
  }
  const int m0 = 0, mx = total_mt;  // the launch's m-tiles
  const int total = mx * P.n_ntiles;
  // Blocks go round-robin over the 8 XCDs (block b to XCD b % 8).  Each
  // round of round_blocks blocks covers that many consecutive tiles of the
  // order (the last round what is left), and XCD x takes the x-th eighth of
  // the round: every XCD gets an equal share of every part of the order
  // (tiles differ in height, so a split of the whole order into eighths
  // would leave some XCDs the heavy groups), and the tiles it runs together
  // are neighbours in the order.
  const int nb = P.round_blocks;
  const int bid = blockIdx.x;
  const int rbase = (bid / nb) * nb;
  const int rs = min(nb, total - rbase);  // tiles in this round
  if (rs <= 0) return;
  const int x = bid & 7, slot = (bid - rbase) >> 3;
  const int L = rbase + (x * rs >> 3) + slot;
  if (L >= rbase + ((x + 1) * rs >> 3)) return;
#if MOE_GEMM_GBAND
  // The part's tiles go group by group, each group's m-tiles in bands of up
  // to GM, n-tile by n-tile: the tiles an XCD runs together are a few
  // m-tiles of one expert by many n-tiles (or of the next expert), so an
  // expert's rows are streamed by few XCDs and every weight panel by one.
  // A group's tiles start at its first m-tile times the n-tiles per m-tile,
  // so the group of tile L is that of m-tile L / n_ntiles.
  const int nn = P.n_ntiles;
  const int q = m0 + L / nn;
  const int g = tile_group[q];
  if (g < 0 || g >= P.G) return;
  const int ga = max(tile_off[g], m0) - m0;            // group's first m-tile in the part
  const int gv = min(tile_off[g + 1], m0 + mx) - m0 - ga;  // its m-tiles in the part
  if (gv <= 0) return;
  const int gr = L - ga * nn;
  const int band = gr / (GM * nn);
  const int gm = min(GM, gv - band * GM);
  const int r = gr - band * GM * nn;
  const int nt = r / gm;
  const int m = m0 + ga + band * GM + (r - nt * gm);
#else
  // The part's tiles go in bands of up to GM m-tiles, n-tile by n-tile, so
  // neighbouring tiles cover a few m-tiles by a few n-tiles and share both
  // operand panels in an XCD's L2.
  const int band = L / (GM * P.n_ntiles);
  const int gm = min(GM, mx - band * GM);
  const int r = L - band * GM * P.n_ntiles;
  const int nt = r / gm;
  const int m = m0 + band * GM + (r - nt * gm);
  const int g = tile_group[m];
  if (g < 0 || g >= P.G) return;
#endif
  const int ml = m - tile_off[g];
  const int gend = group_offsets[g + 1];
  const int row0 = group_offsets[g] + ml * BM;
  if (row0 < 0 || row0 >= gend || gend > P.max_rows) return;
  const int rows = min(BM, gend - row0);
  const int e = P.slot_expert[P.lo_slot + g] - P.e_base;
  if (e < 0 || e >= P.e_res) return;  // rows in a slot that hosts no resident expert
  const int* aidx = P.a_index ? P.a_index + (size_t)pi.j * P.a_index_stride : nullptr;
  // A group's last tile with at most 128 rows runs as a 128-row tile: the
  // same place in the tile order (so it shares the expert's weight panels
  // in L2 with the group's other tiles), half the MFMA work.
  if (HAS_REM && rows <= kRemBM)
    gmm_tile<MOE_GEMM_REM, SWIGLU>(P, smem, aidx, row0, rows, nt, e);
  else if constexpr (BM == 256)
    gmm_tile_pp<SWIGLU, BKM>(P, smem, aidx, row0, rows, nt, e);
  else
    gmm_tile<BM, BK, NST, NW, NWN, SWIGLU>(P, smem, aidx, row0, rows, nt, e);
}

// Both GEMMs of a pass in one launch.  GEMM2 of an m-tile needs every act
// column of that m-tile, that is all GEMM1 n-tiles of it, and nothing else;
// in two launches the chip idles while GEMM1's last short round of tiles
// runs, and again at GEMM2's.  Here the m-tiles are split into 8 contiguous
// runs, one per group of workgroups (block b is in group b % 8, the XCD the
// dispatcher round-robins it to, so a run's weight panels stay in one L2).
// Each workgroup takes one ticket from its group's counter: the group's
// GEMM1 tiles come first (bands of GM m-tiles, n-tile by n-tile), then its
// GEMM2 tiles; tickets past the end exit.  A GEMM1 tile bumps its m-tile's
// count after its act stores, and the tile that completes the count appends
// the m-tile to the group's ready list.  GEMM2 tickets take the m-tiles in
// ready-list order (the i-th n2 tickets: the i-th m-tile to complete), so a
// GEMM2 tile waits only while no further m-tile has completed.  A workgroup
// only ever waits on GEMM1 tiles whose tickets came before its own, held by
// workgroups already running that wait on nothing, so every wait ends (and
// is bounded besides).  sync: [8 groups][16] ints (ticket counter, ready
// count), one count per m-tile, then the ready lists (group v's at its first
// m-tile), all zero at launch.
//
// Visibility of act: GEMM1 stores it write-through (sc1) past its own L2
// and waits for those stores (s_waitcnt 0) before it bumps the m-tile's
// count with a device-scope atomic; the ready entry is stored (agent scope)
// after the last count.  The GEMM2 tile loads with the default policy,
// which is safe because no cache on its side can hold an older copy of
// those rows: its XCD's L2 has not seen them in this launch (they are read
// only after their ready entry is set, the kernel starts with clean caches,
// and nothing else in the launch reads act), and the tile drops its CU's
// L1 (buffer_inv sc0) before loading.  The bumps and the entry are relaxed
// atomics at agent scope: the ordering the reader needs comes from the
// writer's wait for its stores before the bump.
constexpr int kSyncFlags = 128;     // ints before the per-m-tile counts

template <int BM, int BK, int NST, int NW, int NWN>
__global__ __launch_bounds__(64 * NW, 1) void gmm_fused_kernel(GemmParams P1, GemmParams P2,
                                                               int* sync) {
  constexpr bool HAS_REM = BM > kRemBM;
  constexpr int RING = NST * (BM + BNB) * BK * 2;
  static_assert(!HAS_REM || shape_waves(MOE_GEMM_REM) == NW, "REM runs in the same block");
  __shared__ __attribute__((aligned(1024))) char smem[HAS_REM && kRemRing > RING ? kRemRing : RING];
  __shared__ int s_ticket, s_m;
  PassInfo pi = resolve_pass(P1.pa);
  if (!pi.active) return;
  const int* group_offsets = P1.group_offsets + (size_t)pi.j * P1.go_stride;
  const int* tile_off = P1.tile_off + (size_t)pi.j * P1.go_stride;
  const int* tile_group = P1.tile_group + (size_t)pi.j * P1.tg_stride;
  const int M = tile_off[P1.G];
  if (group_offsets[P1.G] > P1.max_rows || M < 0 || M > P1.mt_cap) {  // malformed
    if (blockIdx.x == 0) report(P1.err, MOE_ERR_BAD_OFFSETS);
    return;
  }
  const int v = blockIdx.x & 7;
  const int m0 = (int)(((long long)M * v) >> 3);
  const int mv = (int)(((long long)M * (v + 1)) >> 3) - m0;
  const int n1 = P1.n_ntiles, n2 = P2.n_ntiles;
  const int t1 = mv * n1, tot = t1 + mv * n2;
  if (blockIdx.x / 8 >= tot) return;  // more workgroups than the group's tickets
  const int tid = threadIdx.x;
  if (tid == 0) s_ticket = atomicAdd(sync + v * 16, 1);
  __syncthreads();
  const int t = s_ticket;
  if (t >= tot) return;
  const bool first = t < t1;
  int* ready = sync + kSyncFlags + P1.mt_cap + m0;  // the group's completed m-tiles, + 1
  int m, nt;
  if (first) {
    // GEMM1 tiles in bands of GM m-tiles, n-tile by n-tile
    const int band = t / (GM * n1);
    const int gm = min(GM, mv - band * GM);
    const int r = t - band * GM * n1;
    nt = r / gm;
    m = m0 + band * GM + (r - nt * gm);
  } else {
    // the GEMM2 tiles of the i-th m-tile of the group to complete its GEMM1
    // tiles, n-tile by n-tile
    const int u = t - t1, i = u / n2;
    nt = u - i * n2;
    if (tid == 0) {
      int spins = 0, val = 0;
      if (P1.spin_limit >= 0)
        while ((val = __hip_atomic_load(ready + i, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT)) == 0 &&
               ++spins < P1.spin_limit)
          __builtin_amdgcn_s_sleep(2);
      s_m = val - 1;  // -1 only if the bounded wait ran out
    }
    __syncthreads();
    m = s_m;
    if (m < m0 || m >= m0 + mv) {
      // gave up: these rows of expert_out are not written, and the call
      // says so
      report(P1.err, MOE_ERR_GEMM_WAIT);
      return;
    }
  }
  // the tile's rows and expert (none when the map is malformed or the slot
  // hosts no resident expert: the m-tile's count still counts the tile)
  int row0 = 0, rows = 0, e = -1;
  const int g = tile_group[m];
  if (g >= 0 && g < P1.G) {
    const int gend = group_offsets[g + 1];
    row0 = group_offsets[g] + (m - tile_off[g]) * BM;
    if (row0 >= 0 && row0 < gend && gend <= P1.max_rows) {
      rows = min(BM, gend - row0);
      e = P1.slot_expert[P1.lo_slot + g] - P1.e_base;
      if (e >= P1.e_res) e = -1;
    }
  }
  if (first) {
    if (e >= 0) {
      const int* aidx = P1.a_index ? P1.a_index + (size_t)pi.j * P1.a_index_stride : nullptr;
      if (HAS_REM && rows <= kRemBM)
        gmm_tile<MOE_GEMM_REM, true, true>(P1, smem, aidx, row0, rows, nt, e);
      else
        gmm_tile<BM, BK, NST, NW, NWN, true, true>(P1, smem, aidx, row0, rows, nt, e);
    }
    // every thread's write-through act stores are complete before the count;
    // the m-tile's last GEMM1 tile appends it to the group's ready list
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0 && atomicAdd(sync + kSyncFlags + m, 1) == n1 - 1) {
      const int slot = atomicAdd(sync + v * 16 + 1, 1);
      if (slot < mv)
        __hip_atomic_store(ready + slot, m + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  if (e < 0) return;
  asm volatile("buffer_inv sc0" ::: "memory");  // this CU's L1
  if (HAS_REM && rows <= kRemBM)
    gmm_tile<MOE_GEMM_REM, false>(P2, smem, nullptr, row0, rows, nt, e);
  else
    gmm_tile<BM, BK, NST, NW, NWN, false>(P2, smem, nullptr, row0, rows, nt, e);
}

// fp32 path (the tiny fp32 workload): one thread per output element.
struct F32Params {
  const float* A;
  const int* a_index;
  long long a_index_stride;
  int a_div, a_rows;
  const float* B0;
  const float* B1;
  size_t b_stride;
  float* C;
  const int* group_offsets;
  int go_stride;
  const int* slot_expert;
  int G, K, Nout, lo_slot, e_base, e_res;
  long long max_rows;
  PassArgs pa;
  const int* valid;  // m-tile count of validated offsets (0: compute nothing), or null
};

template <bool SWIGLU>
__global__ __launch_bounds__(256) void gmm_f32_kernel(F32Params P) {
  PassInfo pi = resolve_pass(P.pa);
  if (!pi.active) return;
  const int* go = P.group_offsets + (size_t)pi.j * P.go_stride;
  if (P.valid != nullptr && *P.valid == 0) return;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int row = (int)(idx / P.Nout), col = (int)(idx - (long long)row * P.Nout);
  if (row >= go[P.G] || go[P.G] > P.max_rows) return;
  int lo = 0, hi = P.G;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (go[mid] <= row) lo = mid;
    else hi = mid;
  }
  const int e = P.slot_expert[P.lo_slot + lo] - P.e_base;
  if (e < 0 || e >= P.e_res) return;
  const int src = P.a_index ? P.a_index[(size_t)pi.j * P.a_index_stride + row] / P.a_div : row;
  if (src < 0 || src >= P.a_rows) return;
  const float* a = P.A + (size_t)src * P.K;
  const float* w0 = P.B0 + (size_t)e * P.b_stride + (size_t)col * P.K;
  float s0 = 0.0f, s1 = 0.0f;
  if (SWIGLU) {
    const float* w1 = P.B1 + (size_t)e * P.b_stride + (size_t)col * P.K;
    for (int kk = 0; kk < P.K; ++kk) {
      s0 = fmaf(a[kk], w0[kk], s0);
      s1 = fmaf(a[kk], w1[kk], s1);
    }
    P.C[(size_t)row * P.Nout + col] = s0 / (1.0f + __expf(-s0)) * s1;
  } else {
    for (int kk = 0; kk < P.K; ++kk) s0 = fmaf(a[kk], w0[kk], s0);
    P.C[(size_t)row * P.Nout + col] = s0;
  }
}

// m-tile offsets and the m-tile -> group map from group offsets (standalone
// grouped GEMM calls).  Offsets that are not a non-decreasing sequence
// within [0, min(max_rows, T*k)] give no tiles at all.
__global__ __launch_bounds__(1024) void tile_schedule_kernel(int G, int bm, int limit,
                                                             const int* group_offsets,
                                                             int* tile_off, int* tile_group,
                                                             int* sync, int sync_n, PassArgs pa,
                                                             int* err) {
  PassInfo pi = resolve_pass(pa);
  if (!pi.active) return;
  for (int i = threadIdx.x; i < sync_n; i += blockDim.x) sync[i] = 0;
  __shared__ int tmp[16];
  __shared__ int bad;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int g = threadIdx.x;
  int v = 0;
  if (g < G) {
    int a = group_offsets[g], b = group_offsets[g + 1];
    if (a < 0 || b < a || b > limit) bad = 1;
    v = (b - a + bm - 1) / bm;
  }
  __syncthreads();
  if (bad) v = 0;
  // the first launch of a step call: starts the call's error word
  if (err != nullptr && threadIdx.x == 0) *err = bad ? MOE_ERR_BAD_OFFSETS : 0;
  int x = v;
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) tmp[w] = x;
  __syncthreads();
  if (w == 0) {
    int t = lane < nw ? tmp[lane] : 0;
    for (int off = 1; off < 64; off <<= 1) {
      int y = __shfl_up(t, off);
      if (lane >= off) t += y;
    }
    if (lane < nw) tmp[lane] = t;
  }
  __syncthreads();
  int ex = (w > 0 ? tmp[w - 1] : 0) + x - v;
  if (g < G) {
    tile_off[g] = ex;
    for (int m = 0; m < v; ++m) tile_group[ex + m] = g;
  }
  if (g == 0) tile_off[G] = tmp[nw - 1];
}

// Compute units of the current device rounded down to a multiple of 8 (the
// XCDs): the blocks per round of the tile order.
int round_blocks() {
  static int cus[64] = {0};
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n < 8)
      n = 256;
    cus[dev] = n / 8 * 8;
  }
  return cus[dev];
}

// Workgroups of one tile shape that fit on a CU at once (the GEMM1 kernel).
template <int BM, int BK, int NST, int NW, int NWN>
int resident_blocks() {
  static int occ[64] = {0};
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
  std::lock_guard<std::mutex> lock(mu);
  if (occ[dev] == 0) {
    int n = 0;
    const void* k = reinterpret_cast<const void*>(gmm_bf16_kernel<BM, BK, NST, true, NW, NWN>);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, 64 * NW, 0) != hipSuccess || n < 1)
      n = 1;
    occ[dev] = n;
  }
  return occ[dev];
}

template <int BM, int BK, int NST, int NW, int NWN>
hipError_t launch_bf16(const Dims& d, const PassArgs& pa, const GemmPass& gp, const int* toff,
                       const int* tgroup, int go_stride, int tg_stride, const int* slot_expert,
                       const void* wg, const void* wu, const void* wd, void* act, void* out,
                       int64_t max_rows, int* gsync, hipStream_t s) {
  const long long mt_ub = (max_rows + BM - 1) / BM + d.G_res;
  GemmParams p1;
  p1.A = (const uint16_t*)gp.a_src;
  p1.a_index = gp.a_index;
  p1.a_index_stride = gp.a_index_stride;
  p1.a_div = gp.a_div;
  p1.a_rows = gp.a_src_rows;
  p1.B0 = (const uint16_t*)wg;
  p1.B1 = (const uint16_t*)wu;
  p1.b_stride = (size_t)d.F * d.H;
  p1.C = (uint16_t*)act;
  p1.group_offsets = gp.group_offsets;
  p1.tile_off = toff;
  p1.tile_group = tgroup;
  p1.go_stride = go_stride;
  p1.tg_stride = tg_stride;
  p1.slot_expert = slot_expert;
  p1.G = d.G_res;
  p1.K = d.H;
  p1.Nout = d.F;
  p1.lo_slot = d.lo_slot;
  p1.e_base = d.e_base;
  p1.e_res = d.S_res * d.El;
  p1.max_rows = max_rows;
  p1.n_ntiles = d.F / 128;
  p1.pa = pa;
  GemmParams p2 = p1;
  p2.A = (const uint16_t*)act;
  p2.a_index = nullptr;
  p2.a_index_stride = 0;
  p2.a_div = 1;
  p2.a_rows = (int)max_rows;
  p2.B0 = (const uint16_t*)wd;
  p2.B1 = nullptr;
  p2.b_stride = (size_t)d.H * d.F;
  p2.C = (uint16_t*)out;
  p2.K = d.F;
  p2.Nout = d.H;
  p2.n_ntiles = d.H / 256;
  p1.mt_cap = p2.mt_cap = tile_map_len(d);
  p1.err = p2.err = gp.err;
  p1.spin_limit = p2.spin_limit = gemm_wait_limit();

  if (gsync != nullptr && (MOE_GEMM_FUSE & (BM == 256 ? 2 : 1))) {
    // both GEMMs in one launch (its counters and flags were zeroed before)
    // one workgroup per ticket: 8 groups of up to ceil(mt_ub / 8) m-tiles,
    // GEMM1 and GEMM2 tiles
    const long long nbf = 8 * ((mt_ub + 7) / 8) * (long long)(p1.n_ntiles + p2.n_ntiles);
    p1.round_blocks = p2.round_blocks = 0;
    hipLaunchKernelGGL((gmm_fused_kernel<BM, BK, NST, NW, NWN>), dim3((unsigned)nbf),
                       dim3(64 * NW), 0, s, p1, p2, gsync);
    return hipGetLastError();
  }

  // (Splitting the m-tiles into two GEMM1 -> GEMM2 chains on two streams,
  // so that one half's last GEMM2 round overlaps the other half's work,
  // measured 2-4% slower on the Llama4-Maverick-shaped shard in every mode
  // once the layer's passes hold two chunks: both halves stream the weights
  // of the experts they share.)
  const long long mt = mt_ub + 1;
  const int nb = round_blocks() * resident_blocks<BM, BK, NST, NW, NWN>();
  p1.round_blocks = p2.round_blocks = nb;
  const long long g1 = (mt * p1.n_ntiles + nb - 1) / nb * nb;
  const long long g2 = (mt * p2.n_ntiles + nb - 1) / nb * nb;
  hipLaunchKernelGGL((gmm_bf16_kernel<BM, BK, NST, true, NW, NWN>), dim3((unsigned)g1),
                     dim3(64 * NW), 0, s, p1);
  hipLaunchKernelGGL((gmm_bf16_kernel<BM, BK, NST, false, NW, NWN>), dim3((unsigned)g2),
                     dim3(64 * NW), 0, s, p2);
  return hipGetLastError();
}

}  // namespace

SideStream* side_stream() {
  static SideStream side[64];
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  SideStream& ss = side[dev];
  if (!ss.ok) {
    if (ss.s == nullptr && hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) != hipSuccess)
      return nullptr;
    if (ss.fork == nullptr && hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) != hipSuccess)
      return nullptr;
    if (ss.join == nullptr && hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) != hipSuccess)
      return nullptr;
    ss.ok = true;
  }
  return &ss;
}

std::mutex& side_mutex() {
  static std::mutex mu;
  return mu;
}

namespace {
// ~0.2 s of sleeps: far beyond any tile's own work
constexpr int kDefaultWaitLimit = 1 << 22;
std::atomic<int> g_wait_limit{kDefaultWaitLimit};
}  // namespace

int gemm_wait_limit() { return g_wait_limit.load(std::memory_order_relaxed); }

void set_gemm_wait_limit(int spins) {
  g_wait_limit.store(spins == 0 ? kDefaultWaitLimit : spins, std::memory_order_relaxed);
}

int gmm_sync_ints(const Dims& d) { return kSyncFlags + 2 * tile_map_len(d); }

size_t gmm_sync_bytes(const Dims& d) { return ((size_t)gmm_sync_ints(d) * 4 + 255) / 256 * 256; }

size_t gmm_scratch_bytes(const Dims& d) {
  return ((size_t)(d.G_res + 1) * 4 + 255) / 256 * 256 +
         ((size_t)tile_map_len(d) * 4 + 255) / 256 * 256 + gmm_sync_bytes(d);
}

// C = A B^T over the groups of one pass with the second GEMM's kernel
// (the layer backward's data-gradient products): A [rows, K] read in row
// order, B [e_res][N][K] per resident expert, C [rows, N].  group_offsets
// holds the pass's G_res + 1 offsets (malformed offsets give no tiles).
template <int BM, int BK, int NST, int NW, int NWN>
hipError_t launch_plain(const Dims& d, const int* group_offsets, const int* slot_expert,
                        const void* A, int64_t a_rows, const void* B, size_t b_stride, int K,
                        int N, void* C, int64_t max_rows, void* scratch, hipStream_t s,
                        const void* B1 = nullptr, const void* d_a = nullptr,
                        void* d_h = nullptr, int k_split = 0, const float* row_gate = nullptr,
                        float* dg_part = nullptr) {
  const bool sw = d_h != nullptr;  // the SwiGLU-backward recompute (B, B1: gate, up)
  // k_split > 0: B reduction-major, rows [0, k_split) from B, the rest from B1
  const bool bkm = k_split > 0;
  if (K % BK != 0 || N % (sw ? 128 : 256) != 0 || K <= 0 || N <= 0) return hipErrorNotSupported;
  if (bkm && (BM != 256 || sw || k_split % BK != 0 || k_split > K)) return hipErrorNotSupported;
  int* toff = (int*)scratch;
  int* tgroup = (int*)((char*)scratch + ((size_t)(d.G_res + 1) * 4 + 255) / 256 * 256);
  long long lim = (long long)d.T * d.k;
  if (max_rows < lim) lim = max_rows;
  const PassArgs pa = static_pass_args(0, d.L, 0, 0, d.L);
  hipLaunchKernelGGL(tile_schedule_kernel, dim3(1), dim3(1024), 0, s, d.G_res, BM, (int)lim,
                     group_offsets, toff, tgroup, nullptr, 0, pa, nullptr);
  GemmParams p;
  p.A = (const uint16_t*)A;
  p.a_index = nullptr;
  p.a_index_stride = 0;
  p.a_div = 1;
  p.a_rows = (int)a_rows;
  p.B0 = (const uint16_t*)B;
  p.B1 = (const uint16_t*)B1;
  p.b_stride = b_stride;
  p.C = (uint16_t*)C;
  p.d_a = (const uint16_t*)d_a;
  p.d_h = (uint16_t*)d_h;
  p.k_split = k_split;
  p.row_gate = row_gate;
  p.dg_part = dg_part;
  p.group_offsets = group_offsets;
  p.tile_off = toff;
  p.tile_group = tgroup;
  p.go_stride = 0;
  p.tg_stride = 0;
  p.slot_expert = slot_expert;
  p.G = d.G_res;
  p.K = K;
  p.Nout = N;
  p.lo_slot = d.lo_slot;
  p.e_base = d.e_base;
  p.e_res = d.S_res * d.El;
  p.max_rows = max_rows;
  p.n_ntiles = N / (sw ? 128 : 256);
  p.pa = pa;
  p.mt_cap = tile_map_len(d);
  p.err = nullptr;
  p.spin_limit = gemm_wait_limit();
  const long long mt_ub = (max_rows + BM - 1) / BM + d.G_res;
  const int nb = round_blocks() * resident_blocks<BM, BK, NST, NW, NWN>();
  p.round_blocks = nb;
  const long long g = (mt_ub * p.n_ntiles + nb - 1) / nb * nb;
  if (sw)
    hipLaunchKernelGGL((gmm_bf16_kernel<BM, BK, NST, true, NW, NWN>), dim3((unsigned)g),
                       dim3(64 * NW), 0, s, p);
  else if constexpr (BM == 256) {
    if (bkm)
      hipLaunchKernelGGL((gmm_bf16_kernel<BM, BK, NST, false, NW, NWN, true>), dim3((unsigned)g),
                         dim3(64 * NW), 0, s, p);
    else
      hipLaunchKernelGGL((gmm_bf16_kernel<BM, BK, NST, false, NW, NWN>), dim3((unsigned)g),
                         dim3(64 * NW), 0, s, p);
  } else
    hipLaunchKernelGGL((gmm_bf16_kernel<BM, BK, NST, false, NW, NWN>), dim3((unsigned)g),
                       dim3(64 * NW), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_gmm_plain_kmajor(const Dims& d, const int* group_offsets,
                                   const int* slot_expert, const void* A, int64_t a_rows,
                                   const void* B0, const void* B1, int k_split, size_t b_stride,
                                   int K, int N, void* C, int64_t max_rows, void* scratch,
                                   hipStream_t s) {
  if (!d.bf16 || d.gemm_bm != 256) return hipErrorNotSupported;
  return launch_plain<MOE_GEMM_BIG>(d, group_offsets, slot_expert, A, a_rows, B0, b_stride, K, N,
                                    C, max_rows, scratch, s, B1, nullptr, nullptr, k_split);
}

hipError_t launch_gmm_swiglu_recompute(const Dims& d, const int* group_offsets,
                                       const int* slot_expert, const void* x_sorted,
                                       int64_t a_rows, const void* wg, const void* wu,
                                       const void* d_a, void* d_h, void* act, int64_t max_rows,
                                       void* scratch, hipStream_t s, const float* row_gate,
                                       float* dg_part) {
  if (!d.bf16) return hipErrorNotSupported;
  const size_t fh = (size_t)d.F * d.H;
  if (d.gemm_bm == 256)
    return launch_plain<MOE_GEMM_BIG>(d, group_offsets, slot_expert, x_sorted, a_rows, wg, fh,
                                      d.H, d.F, act, max_rows, scratch, s, wu, d_a, d_h, 0,
                                      row_gate, dg_part);
  return launch_plain<MOE_GEMM_SMALL>(d, group_offsets, slot_expert, x_sorted, a_rows, wg, fh, d.H,
                                      d.F, act, max_rows, scratch, s, wu, d_a, d_h, 0, row_gate,
                                      dg_part);
}

hipError_t launch_gmm_plain(const Dims& d, const int* group_offsets, const int* slot_expert,
                            const void* A, int64_t a_rows, const void* B, size_t b_stride, int K,
                            int N, void* C, int64_t max_rows, void* scratch, hipStream_t s) {
  if (!d.bf16) return hipErrorNotSupported;
  if (d.gemm_bm == 256)
    return launch_plain<MOE_GEMM_BIG>(d, group_offsets, slot_expert, A, a_rows, B, b_stride, K,
                                      N, C, max_rows, scratch, s);
  return launch_plain<MOE_GEMM_SMALL>(d, group_offsets, slot_expert, A, a_rows, B, b_stride, K, N,
                                      C, max_rows, scratch, s);
}

hipError_t launch_gmm(const Dims& d, const PassArgs& pa, const GemmPass& gp,
                      const int* slot_expert, const void* wg, const void* wu, const void* wd,
                      void* act, void* out, int64_t max_rows, void* scratch, hipStream_t s) {
  if (d.bf16) {
    const int* toff = gp.tile_off;
    const int* tgroup = gp.tile_group;
    int go_stride = gp.go_stride, tg_stride = gp.tg_stride;
    int* gsync = gp.sync;
    if (toff == nullptr || tgroup == nullptr) {
      int* t0 = (int*)scratch;
      int* t1 = (int*)((char*)scratch + ((size_t)(d.G_res + 1) * 4 + 255) / 256 * 256);
      long long lim = (long long)d.T * d.k;
      if (max_rows < lim) lim = max_rows;
      // the fused kernel's counters follow the tile map in scratch
      int* t2 = (int*)((char*)t1 + ((size_t)tile_map_len(d) * 4 + 255) / 256 * 256);
      if (gsync == nullptr) gsync = t2;
      hipLaunchKernelGGL(tile_schedule_kernel, dim3(1), dim3(1024), 0, s, d.G_res, d.gemm_bm,
                         (int)lim, gp.group_offsets, t0, t1, gsync == t2 ? t2 : nullptr,
                         gsync == t2 ? gmm_sync_ints(d) : 0, pa, gp.err);
      toff = t0;
      tgroup = t1;
      go_stride = 0;
      tg_stride = 0;
    }
    hipError_t e;
    if (d.gemm_bm == 256)
      e = launch_bf16<MOE_GEMM_BIG>(d, pa, gp, toff, tgroup, go_stride, tg_stride, slot_expert,
                                    wg, wu, wd, act, out, max_rows, gsync, s);
    else
      e = launch_bf16<MOE_GEMM_SMALL>(d, pa, gp, toff, tgroup, go_stride, tg_stride, slot_expert,
                                      wg, wu, wd, act, out, max_rows, gsync, s);
    if (e != hipSuccess) return e;
  } else {
    // a step call validates the offsets (and starts its error word) with
    // the tile schedule; malformed offsets leave no m-tiles, and the
    // kernels then compute nothing
    const int* valid = nullptr;
    if (gp.tile_off == nullptr) {
      int* t0 = (int*)scratch;
      int* t1 = (int*)((char*)scratch + ((size_t)(d.G_res + 1) * 4 + 255) / 256 * 256);
      long long lim = (long long)d.T * d.k;
      if (max_rows < lim) lim = max_rows;
      hipLaunchKernelGGL(tile_schedule_kernel, dim3(1), dim3(1024), 0, s, d.G_res, d.gemm_bm,
                         (int)lim, gp.group_offsets, t0, t1, nullptr, 0, pa, gp.err);
      valid = t0 + d.G_res;
    }
    F32Params p1;
    p1.A = (const float*)gp.a_src;
    p1.a_index = gp.a_index;
    p1.a_index_stride = gp.a_index_stride;
    p1.a_div = gp.a_div;
    p1.a_rows = gp.a_src_rows;
    p1.B0 = (const float*)wg;
    p1.B1 = (const float*)wu;
    p1.b_stride = (size_t)d.F * d.H;
    p1.C = (float*)act;
    p1.group_offsets = gp.group_offsets;
    p1.go_stride = gp.go_stride;
    p1.slot_expert = slot_expert;
    p1.G = d.G_res;
    p1.K = d.H;
    p1.Nout = d.F;
    p1.lo_slot = d.lo_slot;
    p1.e_base = d.e_base;
    p1.e_res = d.S_res * d.El;
    p1.max_rows = max_rows;
    p1.pa = pa;
    p1.valid = valid;
    long long n1 = max_rows * (long long)d.F;
    hipLaunchKernelGGL(gmm_f32_kernel<true>, dim3((unsigned)((n1 + 255) / 256)), dim3(256), 0, s,
                       p1);
    F32Params p2 = p1;
    p2.A = (const float*)act;
    p2.a_index = nullptr;
    p2.a_index_stride = 0;
    p2.a_div = 1;
    p2.a_rows = (int)max_rows;
    p2.B0 = (const float*)wd;
    p2.B1 = nullptr;
    p2.b_stride = (size_t)d.H * d.F;
    p2.C = (float*)out;
    p2.K = d.F;
    p2.Nout = d.H;
    long long n2 = max_rows * (long long)d.H;
    hipLaunchKernelGGL(gmm_f32_kernel<false>, dim3((unsigned)((n2 + 255) / 256)), dim3(256), 0,
                       s, p2);
  }
  return hipGetLastError();
}

}  // namespace moe
