// bfloat16 MFMA contractions of the sparse MoE layer for gfx950.
//
// Sources: "Trainable MoE in CUDA" outline Part 1 (matmul variants X W^T,
// dY W, dY^T X; bias add), Part 3 (gate matmul and its gradient), Part 5
// (expert up/down projections, activation, and the backward for inputs,
// weights and biases); "AI Infra Kernel Lab" README "Project status" (each
// expert's variable-length row segment is tiled independently, empty experts
// and ragged tails handled, no capacity padding) and "Numerical contracts"
// (SwiGLU W2(silu(W1 x) * W3 x)).
//
// One kernel template covers every contraction:
//   * workgroup tile 256 x 256, k-tiles of 32, 256 threads = 4 wavefronts in a
//     2 x 2 grid, each wavefront a 128 x 128 block of 4 x 4 MFMA 32x32x16 tiles
//     with fp32 accumulators; the last m-tile of an expert with at most 128
//     (64) valid rows puts the 4 wavefronts side by side on 64 columns each,
//     4 x 2 (2 x 2) MFMA tiles, so that it costs a fraction of a full tile's
//     MFMA work (the template also holds a 128-row tile with two workgroups per
//     CU for the SGD epilogue, which the persistent form below replaced);
//   * every operand goes straight from global memory into LDS (buffer loads
//     with an LDS destination, bounds checked by the buffer descriptor so
//     ragged rows and k tails read as zero) through a ring of 4 LDS stages,
//     k-tiles loaded 2 ahead of the one in use; the second build of this file
//     (gemm_mfma_kt64.hip, used for the up projection) takes 64-deep k-tiles
//     in 2 LDS stages instead, with the k-tile after next held in registers; K-contiguous operands are kept
//     as [rows][32] (64-byte rows of four 16-byte chunks, chunk XOR-swizzled by
//     (row >> 2) & 3: the LDS has 64 four-byte banks and the 16 lanes served
//     together by a ds_read_b128 read 16 consecutive rows, which then hit 16
//     distinct 16-byte bank groups) and read with ds_read_b128; K-strided
//     operands ([K][M] or [K][N] in memory) keep their natural [k][256] layout
//     and are read with the gfx950 transpose read ds_read_b64_tr_b16, so the
//     MFMA loop is the same for every layout;
//   * each k-step is 16 issue slots of one MFMA followed by either one
//     fragment read for the next k-step or one load of a later k-tile, so
//     neither the LDS nor the load queue ever holds up a run of MFMAs; one
//     barrier per k-tile publishes the next stage, with the first fragments of
//     that stage read under the last MFMAs of the current one;
//   * the MFMA is issued with the N operand first, so each lane's
//     accumulators hold 4 consecutive output columns; every epilogue goes
//     out through LDS, so that each store instruction writes whole rows with
//     16-byte vectors: plain stores (bf16 or fp32) and the SwiGLU forward in
//     one or two passes, and the MLP forward (bias + activation), the
//     activation backward (H in, dH out) and the fused SGD step (masters in
//     and out, bf16 copies out) in 32-row passes whose global loads and stores
//     go through buffer descriptors, issued unconditionally so that the wait
//     counts stay exact;
//   * tiles are scheduled on the device from the expert offsets: ROWS mode
//     walks the m-tiles of every expert's row segment (prefix of per-expert
//     tile counts, binary search per workgroup); KSEG mode gives each expert
//     its own output and runs K over its row segment (empty segment -> the
//     output is written as zeros); DENSE is one plain GEMM, or with kchunk
//     set, one fp32 partial output per K segment (summed afterwards in
//     segment order).  The hardware
//     deals workgroups round-robin to the 8 XCDs; the kernel groups the XCDs
//     (G per group) and gives each group a contiguous, equal share of the
//     tiles (in KSEG mode, of each segment's tiles, since a tile's cost there
//     follows its segment's row count), dealt round-robin among its members;
//   * the weight gradients with the SGD step run persistent: one workgroup per CU
//     loops over tiles taken from its XCD group's queue (one integer atomic per
//     tile), segments with the most rows first;
//   * gathered operands (fused dispatch): A rows of a row-mode contraction, or the
//     k-rows of a weight gradient's operand, come from a token-major source
//     through token_of; a weight gradient's k-row indices reach LDS through a
//     small ring two k-tiles ahead of the operand loads that use them.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {
#ifdef MOE_GEMM_KT64
namespace kt64 {
#endif

#ifdef MOE_GEMM_KT64
// the second build of this file (gemm_mfma_kt64.hip): 64-deep k-tiles, so a K-contiguous
// operand row of a k-tile is one whole 128-byte line, with loads staged through registers
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int NS = 2;                           // LDS stages
constexpr int DIST = 1;
#else
constexpr int BM = 256, BN = 256, BK = 32;
constexpr int NS = 4;                           // LDS stages (ring)
constexpr int DIST = 2;                         // k-tiles loaded ahead of the one in use
#endif
constexpr int NTHR = 256;
constexpr int KSTEPS = BK / 16;                 // MFMA k-steps per k-tile
constexpr int TILE_ELEMS = 256 * BK;            // one operand tile in LDS (bf16)
constexpr int CHUNKS = BK / 8;                  // 16-byte chunks per K-contiguous row
constexpr int ROWS_PER_WIN = 256 / (BK * 2);    // rows per 256-byte bank window
constexpr int DIRECT_ROWS = 1024 / (BK * 2);    // K-contiguous rows filled by one wave load
constexpr int DIRECT_IPW = 256 / DIRECT_ROWS / 4;   // loads per wave per operand tile
constexpr int STRIDED_IPW = BK / 2 / 4;             // K-strided: two k-rows per load
constexpr int GROUP_N = 8;                      // n-tiles per tile group (L2 reuse)
static_assert(DIST >= 1 && DIST <= NS - 1, "prefetch distance");
static_assert(NS * 2 * TILE_ELEMS * 2 <= 160 * 1024, "LDS");

enum { MODE_ROWS = 0, MODE_KSEG = 1, MODE_DENSE = 2 };

typedef __amdgpu_buffer_rsrc_t rsrc_t;

struct GemmParams {
    const bf16* A; long lda;
    const bf16* B; const bf16* B2; long ldb; long bes;
    int b2_kstart;
    int paired;
    int M, N, K, E;
    const int32_t* offsets;
    const int32_t* tile_prefix;
    int mtiles_ub;
    int kchunk;                   // KSEG without offsets: segment e is rows [e kchunk, (e+1) kchunk) of K
    int xcd_group;                // XCDs per tile group: 1, 2, 4 or 8 (see the tile deal)
    void* C; void* C2; long ldc; long ces;
    int c2_mstart;
    void* W; void* W2; float lr;  // EPI_SGD: C/C2 are fp32 masters, W/W2 their bf16 copies
    const bf16* bias; long bias_es;
    const bf16* H; long ldh; int ffn;
    // gathered operand rows (fused dispatch): token index of each expert-major row
    const int32_t* rows_tok;      // GA_ROWS: rows of A; GA_KA / GA_KB: k-rows of A / B
    int src_rows;                 // rows of the token-major source the gathered rows come from
    const float* row_scale;       // EPI_UP_SWIGLU_G / EPI_DN_SWIGLU_G: gate of each expert-major row
    float* dot_part;              // EPI_DN_SWIGLU_G: [N-tiles][rows] partial <dA, A> of each row
    long dot_ld;                  // rows of dot_part per N-tile
    // EPI_SCATTER: the expert-major rows of dX (slot_of[t k + i] is token t's i-th), and the
    // shared branch's part [T, d] or NULL
    const bf16* scat_rows; const int32_t* scat_slot; const bf16* scat_shared;
    // persistent weight gradients: one tile counter per XCD group (zeroed before the launch),
    // and the segments in the order their tiles are handed out (most rows first)
    int32_t* queue;
    const int32_t* seg_order;
};
// Gathered operands.  GA_ROWS: the K-contiguous A operand of a row-mode contraction is
// read from rows rows_tok[p] of a token-major source instead of rows p of an expert-major
// one.  GA_KA / GA_KB: the k-strided A / B operand of a weight gradient takes its k-row p
// (a row of the expert's segment) from row rows_tok[p] of a token-major source.
enum { GA_NONE = 0, GA_ROWS = 1, GA_KA = 2, GA_KB = 3 };

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, long bytes) {
    if (bytes < 0) bytes = 0;
    if (bytes > 0x7fffffffL) bytes = 0x7fffffffL;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
typedef __attribute__((address_space(3))) void* lds_ptr_t;
__device__ __forceinline__ void bload_lds(rsrc_t r, const bf16* lds, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(lds), 16, voff, soff, 0, 0);
}
// s_waitcnt with only vmcnt constrained / only lgkmcnt constrained
template <int N> __device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); }

// Sum over each half (32 lanes) of the wavefront, the same value on every lane of the half:
// DPP quad swaps and row mirrors leave each 16-lane row holding its sum, then the two rows
// of each half are added in a fixed order.
template <int C> __device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), C, 0xF, 0xF, false));
}
__device__ __forceinline__ float half_wave_sum(float v) {
    v += dpp_f<0xB1>(v);          // quad lane ^ 1
    v += dpp_f<0x4E>(v);          // quad lane ^ 2
    v += dpp_f<0x141>(v);         // half-row mirror
    v += dpp_f<0x140>(v);         // row mirror
    const float lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
                     __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)) +
                     __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (threadIdx.x & 32) ? hi : lo;
}

// One wave load: 64 lanes x 16 bytes from a buffer straight into LDS at lds_addr + lane * 16.
// Issued through inline assembly so that the compiler's wait-count insertion does not
// turn every later LDS read into a full drain of the load queue: the kernel counts
// these loads itself (s_waitcnt vmcnt) before the barrier that publishes a stage.
// M0 (the LDS destination register) is written here and used by nothing else in
// these kernels; it is listed as clobbered, which clang reports as a reserved register.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(rsrc_t r, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(lds_addr), "v"(voff), "s"(r), "s"(soff) : "memory", "m0");
}
// The same for 4 bytes a lane (the k-row token indices of a gathered weight-gradient operand).
__device__ __forceinline__ void dma4(rsrc_t r, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :: "s"(lds_addr), "v"(voff), "s"(r), "s"(soff) : "memory", "m0");
}
#pragma clang diagnostic pop
// Where this wave's loads of one operand tile come from.  K-contiguous operands:
// load i fills DIRECT_ROWS rows (lane -> row lane / CHUNKS, physical chunk lane % CHUNKS,
// holding the logical chunk that the swizzle puts there); K-strided operands: load i
// fills k-rows 2j, 2j + 1 of a natural [k][256] tile.
struct OpPlan {
    rsrc_t r0, r1;          // r1: second source (paired rows, or k >= kswitch)
    uint32_t ld_bytes;
    int paired, kswitch, strided;
    uint32_t vo[2];         // lane offsets for even / odd loads
};
__device__ __forceinline__ OpPlan plan_direct(rsrc_t r0, rsrc_t r1, uint32_t ld, int paired) {
    OpPlan o;
    o.r0 = r0; o.r1 = r1; o.ld_bytes = ld; o.paired = paired; o.kswitch = 0x7fffffff; o.strided = 0;
    const int lane = threadIdx.x & 63;
    const uint32_t row_off = (uint32_t)(lane / CHUNKS) * ld;
#pragma unroll
    for (int par = 0; par < 2; ++par) {
        const int key = (((DIRECT_ROWS * par) + lane / CHUNKS) / ROWS_PER_WIN) & (CHUNKS - 1);
        o.vo[par] = row_off + ((uint32_t)((lane % CHUNKS) ^ key) << 4);
    }
    return o;
}
// K-strided operand [k][W columns], W = 256 (two k-rows per wave load) or 128 (four):
// 16-byte chunk c of k-row r sits at chunk c ^ 2 (r & 3) of its LDS row
template <int W = 256>
__device__ __forceinline__ OpPlan plan_strided(rsrc_t r0, rsrc_t r1, uint32_t ld, int kswitch) {
    OpPlan o;
    o.r0 = r0; o.r1 = r1; o.ld_bytes = ld; o.paired = 0; o.kswitch = kswitch; o.strided = 1;
    const int lane = threadIdx.x & 63;
    if (W == 256) {
        const uint32_t row_off = (uint32_t)(lane >> 5) * ld;
        o.vo[0] = row_off + ((uint32_t)((lane & 31) ^ (2 * (lane >> 5))) << 4);
        o.vo[1] = row_off + ((uint32_t)((lane & 31) ^ (4 + 2 * (lane >> 5))) << 4);
    } else {
        const uint32_t r = (uint32_t)(lane >> 4);
        o.vo[0] = o.vo[1] = r * ld + ((uint32_t)((lane & 15) ^ (2 * r)) << 4);
    }
    return o;
}
// load i (0 .. IPW-1) of this wave for k-tile starting at k0, into the tile at lds byte address t
template <bool STRIDED, int W = 256>
__device__ __forceinline__ void dma_one(const OpPlan& o, int i, uint32_t t, int k0, int wave) {
    if (STRIDED) {
        constexpr int RPL = 512 / W;                  // k-rows per wave load
        constexpr int IPW = BK / RPL / 4;              // loads per wave per k-tile
        const int j = wave * IPW + i;
        rsrc_t r = o.r0;
        int kk = k0;
        if (k0 >= o.kswitch) { r = o.r1; kk = k0 - o.kswitch; }
        dma16(r, t + j * 1024, o.vo[i & 1], (uint32_t)(kk + RPL * j) * o.ld_bytes);
    } else {                                          // W tile rows
        const int j = wave * (W / DIRECT_ROWS / 4) + i;
        const int row0 = DIRECT_ROWS * j;
        int rowbase = row0;
        rsrc_t r = o.r0;
        if (o.paired) {      // tile rows alternate 32 W1 rows and the 32 W3 rows of the same units
            rowbase = ((row0 >> 6) << 5) + (row0 & 31);
            if ((row0 >> 5) & 1) r = o.r1;
        }
        dma16(r, t + j * 1024, o.vo[i & 1], (uint32_t)rowbase * o.ld_bytes + (uint32_t)k0 * 2u);
    }
}

#ifdef MOE_GEMM_KT64
typedef unsigned int nu4r __attribute__((ext_vector_type(4)));
// The 16 bytes a lane's dma_one would bring, loaded into registers instead.
template <bool STRIDED, int W = 256>
__device__ __forceinline__ nu4r load_one(const OpPlan& o, int i, int k0, int wave) {
    if (STRIDED) {
        constexpr int RPL = 512 / W;
        constexpr int IPW = BK / RPL / 4;
        const int j = wave * IPW + i;
        rsrc_t r = o.r0;
        int kk = k0;
        if (k0 >= o.kswitch) { r = o.r1; kk = k0 - o.kswitch; }
        return __builtin_bit_cast(nu4r, __builtin_amdgcn_raw_buffer_load_b128(
            r, o.vo[i & 1], (uint32_t)(kk + RPL * j) * o.ld_bytes, 0));
    } else {
        const int j = wave * (W / DIRECT_ROWS / 4) + i;
        const int row0 = DIRECT_ROWS * j;
        int rowbase = row0;
        rsrc_t r = o.r0;
        if (o.paired) {
            rowbase = ((row0 >> 6) << 5) + (row0 & 31);
            if ((row0 >> 5) & 1) r = o.r1;
        }
        return __builtin_bit_cast(nu4r, __builtin_amdgcn_raw_buffer_load_b128(
            r, o.vo[i & 1], (uint32_t)rowbase * o.ld_bytes + (uint32_t)k0 * 2u, 0));
    }
}
#endif

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s* lds_v4s_ptr;
template <int W = 256>
__device__ __forceinline__ bf16x8 read_strided(const bf16* T, int colbase, int ks) {
    const int lane = threadIdx.x & 63;
    const int L = lane & 15;
    const int col = colbase + 16 * ((lane >> 4) & 1) + 4 * (L & 3);
    const int pc = (col >> 3) ^ (2 * (L >> 2));
    const int k = 16 * ks + 8 * (lane >> 5) + (L >> 2);
    const bf16* p0 = T + k * W + pc * 8 + (col & 7);
    const bf16* p1 = p0 + 4 * W;
    v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(p0));
    v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(p1));
    typedef short v8s __attribute__((ext_vector_type(8)));
    v8s v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}
struct Frags { bf16x8 a[4], b[4]; };
template <int I, int J> struct Layout { static constexpr int NI = I, NJ = J; };
__device__ __forceinline__ bf16x8 read_contig(const bf16* T, int rowbase, int ks) {
    const int lane = threadIdx.x & 63;
    const int rr = lane & 31, hk = lane >> 5;
    const int key = ((rowbase + rr) / ROWS_PER_WIN) & (CHUNKS - 1);
    const int ch = ((2 * ks + hk) ^ key) << 3;
    return *reinterpret_cast<const bf16x8*>(T + (rowbase + rr) * BK + ch);
}
typedef float nf4 __attribute__((ext_vector_type(4)));
typedef unsigned int nu2 __attribute__((ext_vector_type(2)));
typedef unsigned int nu4 __attribute__((ext_vector_type(4)));
// 8 bf16 of a 16-byte vector to float, and back (round to nearest even)
__device__ __forceinline__ void unpack8(nu4 u, float* f) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        f[2 * k] = __uint_as_float(u[k] << 16);
        f[2 * k + 1] = __uint_as_float(u[k] & 0xffff0000u);
    }
}
__device__ __forceinline__ nu4 pack8(const float* f) {
    nu4 u;
    bf16* b = reinterpret_cast<bf16*>(&u);
#pragma unroll
    for (int k = 0; k < 8; ++k) b[k] = (bf16)f[k];
    return u;
}
__device__ __forceinline__ void store4(bf16* p, const float* v) {
    uint2 u;
    bf16* b = reinterpret_cast<bf16*>(&u);
    b[0] = (bf16)v[0]; b[1] = (bf16)v[1]; b[2] = (bf16)v[2]; b[3] = (bf16)v[3];
    *reinterpret_cast<uint2*>(p) = u;
}
__device__ __forceinline__ void store4(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void load4(const bf16* p, float* v) {
    uint2 u = *reinterpret_cast<const uint2*>(p);
    const bf16* b = reinterpret_cast<const bf16*>(&u);
    v[0] = (float)b[0]; v[1] = (float)b[1]; v[2] = (float)b[2]; v[3] = (float)b[3];
}
__device__ __forceinline__ void grouped(int q, int mt, int nt, int& tm, int& tn) {
    const int gn = min(GROUP_N, nt);
    const int ng = q / (mt * gn);
    const int rem = q - ng * mt * gn;
    const int gsz = min(gn, nt - ng * gn);
    tm = rem / gsz;
    tn = ng * gn + (rem - tm * gsz);
}

// Shared memory of one tile: the ring of operand stages, then (gathered k-rows) the ring of
// their token indices, then (scatter epilogue) the slots of the tile's rows.
template <int EPI, int TM, int GA>
struct TileLds {
    static constexpr bool KGATHER = GA == GA_KA || GA == GA_KB;
    static constexpr int NSt = TM == 128 ? 3 : NS;
    static constexpr int TILE_A = TM * BK, STAGE = TILE_A + TILE_ELEMS;
    // KGATHER: after the stages, a ring of NSt slots of k-row token indices, 256 bytes per
    // wavefront (its 8 k-rows of a k-tile, in the order it reads them)
    static constexpr int IDX_ELEMS = KGATHER ? NSt * 512 : 0;
    // EPI_SCATTER: after the stages, the slots of the tile's 256 rows (8 KB)
    static constexpr int SCAT_ELEMS = EPI == EPI_SCATTER ? 256 * MOE_SCATTER_FUSED_K * 2 : 0;
    static constexpr int ELEMS = NSt * STAGE + IDX_ELEMS + SCAT_ELEMS;
};

// One output tile L of a contraction (L indexes the contraction's tiles as the schedule
// below lays them out), from its k-loop to its epilogue, with the workgroup's shared
// memory at lds (TileLds<EPI, TM, GA>::ELEMS elements).  TM: tile rows.  256: one
// workgroup per CU, a 4-stage ring; 128 (the SGD epilogue of the weight gradients): two
// workgroups per CU, 128 accumulators a lane and a 3-stage ring.
template <int MODE, bool AT, bool BT, int EPI, bool OUT_F32, int TM = 256, int GA = GA_NONE>
__device__ __forceinline__ void gemm_tile(const GemmParams& p, int L, bf16* lds) {
    static_assert(TM == 256 || (TM == 128 && ((MODE == MODE_KSEG && EPI == EPI_SGD) || MODE == MODE_ROWS)),
                  "128-row tiles: SGD epilogue or row mode");
    constexpr int AIPW = TM / DIRECT_ROWS / 4;       // K-contiguous A loads per wave per tile
    static_assert(GA == GA_NONE || (GA == GA_ROWS && MODE == MODE_ROWS && !AT) ||
                  (GA == GA_KA && MODE == MODE_KSEG && AT && TM == 256) ||
                  (GA == GA_KB && MODE == MODE_KSEG && BT), "gathered operand");
    using S = TileLds<EPI, TM, GA>;
    constexpr bool KGATHER = S::KGATHER;
#ifdef MOE_GEMM_KT64
    static_assert(!KGATHER, "k-row gathers run in the 32-deep build");
#endif
    constexpr int NSt = S::NSt, TILE_A = S::TILE_A, STAGE = S::STAGE, IDX_ELEMS = S::IDX_ELEMS;
    static_assert(DIST <= NSt - 1, "prefetch distance");
    const int tid = threadIdx.x, lane = tid & 63, wave = uni(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int NT = p.paired ? (p.ffn + 127) / 128 : (p.N + BN - 1) / BN;

    int e = 0, m0 = 0, n_t = 0;
    long row_base = 0;
    int rows_valid = 0;
    int K = p.K;
    int kbase = 0;                 // DENSE split over K: first column of this segment's K range
    if (MODE == MODE_ROWS) {
        const int tmg = L / NT;
        int lo = 0, hi = p.E;
        while (hi - lo > 1) {
            int mid = (lo + hi) >> 1;
            if (p.tile_prefix[mid] <= tmg) lo = mid; else hi = mid;
        }
        e = lo;
        const int mt = p.tile_prefix[e + 1] - p.tile_prefix[e];
        int tm;
        grouped(L - p.tile_prefix[e] * NT, mt, NT, tm, n_t);
        m0 = tm * TM;
        row_base = p.offsets[e];
        const int seg = p.offsets[e + 1] - p.offsets[e];
        rows_valid = min(TM, seg - m0);
    } else if (MODE == MODE_KSEG) {
        const int MT = (p.M + TM - 1) / TM;
        e = L / (MT * NT);
        int tm;
        grouped(L - e * MT * NT, MT, NT, tm, n_t);
        m0 = tm * TM;
        rows_valid = min(TM, p.M - m0);
        if (p.offsets) {
            row_base = p.offsets[e];
            K = p.offsets[e + 1] - p.offsets[e];
        } else if (p.kchunk > 0) {
            row_base = (long)e * p.kchunk;
            K = min(p.kchunk, p.K - (int)row_base);
        }
    } else {
        const int MT = (p.M + BM - 1) / BM;
        int tm, Lt = L;
        if (p.kchunk > 0) {        // segment e: K columns [e kchunk, min((e+1) kchunk, K))
            e = L / (MT * NT);
            Lt = L - e * MT * NT;
            kbase = e * p.kchunk;
            K = min(p.kchunk, p.K - kbase);
        }
        grouped(Lt, MT, NT, tm, n_t);
        m0 = tm * BM;
        rows_valid = min(BM, p.M - m0);
    }
    e = uni(e); m0 = uni(m0); n_t = uni(n_t); rows_valid = uni(rows_valid); K = uni(K); kbase = uni(kbase);
    row_base = (long)uni((int)row_base);
    const int n0 = n_t * BN;
    const int hid0 = n_t * 128;
    const bf16* Be = p.B + (long)e * p.bes;
    const bf16* B2e = p.B2 ? p.B2 + (long)e * p.bes : nullptr;

    constexpr uint32_t OUTB = 0x80000000u;         // a byte offset past every buffer bound
    OpPlan pa, pb;
    // GA_ROWS: lane offset of each of this wave's A loads, the gathered row's start plus the
    // swizzled chunk (OUTB for rows past the tile: they read zeros)
    uint32_t gvo[GA == GA_ROWS ? AIPW : 1];
    if (AT) {   // A[k][m]
        if constexpr (GA == GA_KA) {      // k-row p is row rows_tok[p] of the source
            rsrc_t r = make_rsrc(p.A + m0, ((long)p.src_rows * p.lda - m0) * 2);
            pa = plan_strided<TM>(r, r, (uint32_t)(p.lda * 2), 0x7fffffff);
        } else {
            const bf16* base = p.A + row_base * p.lda + m0;
            rsrc_t r = make_rsrc(base, ((long)K * p.lda - m0) * 2);
            pa = plan_strided<TM>(r, r, (uint32_t)(p.lda * 2), 0x7fffffff);
        }
    } else if constexpr (GA == GA_ROWS) {   // A[m][k], row m of the tile = source row rows_tok[m]
        rsrc_t r = make_rsrc(p.A, (long)p.src_rows * p.lda * 2);
        pa = plan_direct(r, r, (uint32_t)(p.lda * 2), 0);
        const int lr = lane / CHUNKS;
#pragma unroll
        for (int i = 0; i < AIPW; ++i) {
            const int row = DIRECT_ROWS * (wave * AIPW + i) + lr;
            const uint32_t chunk = pa.vo[i & 1] - (uint32_t)lr * pa.ld_bytes;
            gvo[i] = row < rows_valid ? (uint32_t)p.rows_tok[row_base + m0 + row] * pa.ld_bytes + chunk : OUTB;
        }
    } else {    // A[m][k]
        const bf16* base = p.A + (row_base + m0) * p.lda + kbase;
        rsrc_t r = make_rsrc(base, ((long)rows_valid * p.lda - kbase) * 2);
        pa = plan_direct(r, r, (uint32_t)(p.lda * 2), 0);
    }
    if (BT) {   // B[k][n]
        if (GA == GA_KB) {                // k-row p is row rows_tok[p] of the source
            rsrc_t r = make_rsrc(p.B + n0, ((long)p.src_rows * p.ldb - n0) * 2);
            pb = plan_strided(r, r, (uint32_t)(p.ldb * 2), 0x7fffffff);
        } else if (MODE == MODE_KSEG) {
            const bf16* base = p.B + row_base * p.ldb + n0;
            rsrc_t r = make_rsrc(base, ((long)K * p.ldb - n0) * 2);
            pb = plan_strided(r, r, (uint32_t)(p.ldb * 2), 0x7fffffff);
        } else if (p.b2_kstart >= 0) {
            pb = plan_strided(make_rsrc(Be + n0, ((long)p.b2_kstart * p.ldb - n0) * 2),
                              make_rsrc(B2e + n0, ((long)(K - p.b2_kstart) * p.ldb - n0) * 2),
                              (uint32_t)(p.ldb * 2), p.b2_kstart);
        } else {
            rsrc_t r = make_rsrc(Be + n0, ((long)K * p.ldb - n0) * 2);
            pb = plan_strided(r, r, (uint32_t)(p.ldb * 2), 0x7fffffff);
        }
    } else {    // B[n][k]
        if (p.paired)
            pb = plan_direct(make_rsrc(Be + (long)hid0 * p.ldb, (long)(p.ffn - hid0) * p.ldb * 2),
                             make_rsrc(B2e + (long)hid0 * p.ldb, (long)(p.ffn - hid0) * p.ldb * 2),
                             (uint32_t)(p.ldb * 2), 1);
        else {
            rsrc_t r = make_rsrc(Be + (long)n0 * p.ldb + kbase, ((long)min(BN, p.N - n0) * p.ldb - kbase) * 2);
            pb = plan_direct(r, r, (uint32_t)(p.ldb * 2), 0);
        }
    }

    constexpr int NIMAX = TM / 64;                    // MFMA row blocks per wave
    f32x16 acc[NIMAX][4];
#pragma unroll
    for (int i = 0; i < NIMAX; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    constexpr int IPW_A = AT ? BK / (512 / TM) / 4 : AIPW;
    constexpr int IPW_B = BT ? STRIDED_IPW : DIRECT_IPW;
    constexpr int LPW = IPW_A + IPW_B;                 // loads per wave per k-tile
    // each k-step issues PART loads in its MFMA slots; the narrowest wave layout (2 x 2)
    // has 4 slots a k-step, so PART <= 4 keeps every load of a k-tile issued
    static_assert(LPW % KSTEPS == 0 && LPW / KSTEPS <= 4, "load parts");
    constexpr int PART = LPW / KSTEPS;
    const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds;
    const int nk = (K + BK - 1) / BK;
    // load q (0 .. LPW-1) of k-tile kt; tiles past the end load harmless data (the buffer
    // bounds make them zeros or rows of this operand) into a stage nobody reads again
    // KGATHER: the token indices of k-tile kt's k-rows reach LDS one k-tile before that
    // k-tile's operand loads are issued (ring slot kt % NSt; wave w's 8 k-rows 8w..8w+7 of
    // the k-tile, stored so that lane half h reads the indices of its k-rows 8w + 2i + h,
    // i = 0..3, as one 16-byte vector); tk holds those of the k-tile being loaded
    uint32_t tk[KGATHER ? STRIDED_IPW : 1];
    const uint32_t idx_base = lds_base + (uint32_t)(NSt * STAGE * 2);
    const rsrc_t ridx = make_rsrc(KGATHER ? p.rows_tok + row_base : nullptr, KGATHER ? (long)K * 4 : 0);
    auto idx_dma = [&](int kt) {
        const int l = lane & 7;
        dma4(ridx, idx_base + (uint32_t)(kt % NSt) * 1024u + (uint32_t)wave * 256u,
             (uint32_t)(2 * (l & 3) + ((l >> 2) & 1)) * 4u, (uint32_t)(kt * BK + 8 * wave) * 4u);
    };
    auto idx_read = [&](int kt) {
        const nu4 v = *reinterpret_cast<const nu4*>(reinterpret_cast<const char*>(lds) + NSt * STAGE * 2 +
                                                    (kt % NSt) * 1024 + wave * 256 + (lane >> 5) * 16);
#pragma unroll
        for (int i = 0; i < (KGATHER ? STRIDED_IPW : 1); ++i) tk[i] = v[i];
    };
    // load i of a gathered k-strided operand: k-row kt BK + 2 (wave IPW + i) + h of the
    // segment, read from its source row (k-rows past the segment read zeros)
    auto dma_gathered = [&](const OpPlan& o, int i, uint32_t t, int kt) {
        const int h = lane >> 5;
        const int j = wave * STRIDED_IPW + i;
        const uint32_t chunk = o.vo[i & 1] - (uint32_t)h * o.ld_bytes;
        const uint32_t voff = (kt * BK + 2 * j + h < K) ? tk[i] * o.ld_bytes + chunk : OUTB;
        dma16(o.r0, t + (uint32_t)j * 1024u, voff, 0);
    };
    auto dma = [&](int q, int kt) {
        const uint32_t st = (uint32_t)(kt % NSt) * (STAGE * 2);
        if (q < IPW_A) {
            if constexpr (GA == GA_ROWS)
                dma16(pa.r0, lds_base + st + (uint32_t)(wave * AIPW + q) * 1024u, gvo[q], (uint32_t)(kt * BK) * 2u);
            else if constexpr (GA == GA_KA) dma_gathered(pa, q, lds_base + st, kt);
            else dma_one<AT, TM>(pa, q, lds_base + st, kt * BK, wave);
        } else {
            if constexpr (GA == GA_KB) dma_gathered(pb, q - IPW_A, lds_base + st + TILE_A * 2, kt);
            else dma_one<BT>(pb, q - IPW_A, lds_base + st + TILE_A * 2, kt * BK, wave);
        }
    };
    const int rr = lane & 31, hk = lane >> 5;

    // The main loop and epilogue for one wave layout (NI x NJ MFMA blocks per wave):
    // 4 x 4 with the waves in a 2 x 2 grid of 128 x 128; for row tiles with at most 128
    // (64) valid rows, 4 x 2 (2 x 2) with the waves side by side on 64 columns each, so
    // that a short tail tile costs a fraction of the MFMA work of a full one.
    auto tile = [&](auto lay) {
        constexpr int NI = decltype(lay)::NI, NJ = decltype(lay)::NJ;
        constexpr int NMF = NI * NJ;                   // MFMA slots per k-step
        constexpr int NR = NI + NJ;                    // fragment reads per k-step
        const int rb = (NJ == 4) ? wm * (NI * 32) : 0;  // first row / column of the wave
        const int cb = (NJ == 4) ? wn * 128 : wave * 64;
        // fragment read idx of a k-step, in the order the MFMAs use them: a0, then b0 .. b(NJ-1)
        // (the first row of MFMAs), then a1 .. a(NI-1), so that each MFMA waits only for
        // the reads it needs and not for the whole step's
        auto read_one = [&](const bf16* As, const bf16* Bs, int ks, Frags& f, int idx) {
            const int ia = idx == 0 ? 0 : idx - NJ, ib = idx - 1;
            if (idx == 0 || idx > NJ) f.a[ia] = AT ? read_strided<TM>(As, rb + ia * 32, ks) : read_contig(As, rb + ia * 32, ks);
            else f.b[ib] = BT ? read_strided(Bs, cb + ib * 32, ks) : read_contig(Bs, cb + ib * 32, ks);
        };
        auto mfma_one = [&](const Frags& f, int i) {
            const int ii = i / NJ, jj = i % NJ;
            acc[ii][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[jj], f.a[ii], acc[ii][jj], 0, 0, 0);
        };

        // EPI_SGD: the tile's fp32 masters (and bf16 copies), and its first two passes of
        // masters loaded before the main loop (they arrive with the first k-tile's loads)
        const int qt = tid & 63, rs = wave;            // a wavefront updates whole rows
        const int n = n0 + qt * 4;
        const bool col_ok = n < p.N;
        const float nlr = -p.lr;
        float* const M1 = reinterpret_cast<float*>(p.C);
        float* const M2 = reinterpret_cast<float*>(p.C2);
        bf16* const W1 = reinterpret_cast<bf16*>(p.W);
        bf16* const W2 = reinterpret_cast<bf16*>(p.W2);
        const int c2 = M2 ? p.c2_mstart : 0x7fffffff;
        const long ldc = p.ldc, eoff = (long)e * p.ces;
        // Tile rows [0, n1) are rows m0.. of C (W), rows [n1, rows_valid) rows of C2 (W2).
        // One buffer descriptor per half bounds the tile's rows up to column N, so that
        // every load and store is issued unconditionally (exact wait counts) and a lane
        // outside the tile gets an offset past the bound: its store is dropped and its
        // load returns zeros.
        const int n1 = max(0, min(rows_valid, c2 - m0));
        const int n2 = rows_valid - n1;
        const long b1 = eoff + (long)m0 * ldc, b2 = eoff + (long)max(m0 - c2, 0) * ldc;
        const rsrc_t rm1 = make_rsrc(M1 + b1, n1 > 0 ? ((long)(n1 - 1) * ldc + p.N) * 4 : 0);
        const rsrc_t rw1 = make_rsrc(W1 + b1, n1 > 0 ? ((long)(n1 - 1) * ldc + p.N) * 2 : 0);
        const rsrc_t rm2 = n2 > 0 ? make_rsrc(M2 + b2, ((long)(n2 - 1) * ldc + p.N) * 4) : rm1;
        const rsrc_t rw2 = n2 > 0 ? make_rsrc(W2 + b2, ((long)(n2 - 1) * ldc + p.N) * 2) : rw1;
        constexpr uint32_t OUT = 0x80000000u;          // past every bound
        // element offset of tile row ml (wave-uniform) at this thread's columns in its
        // half, or OUT
        // mo: the row's offset in the tile less this wavefront's rs.  The row and its half are
        // worked out afresh at each use (rs and n1 pass through an empty asm): otherwise the
        // compiler computes all 64 rows' indices and descriptor choices once, for the load two
        // passes ahead and for the store, and keeps hundreds of copies live in (and spilled
        // out of) the scalar registers through the whole epilogue.
        auto elem = [&](int mo, bool& sec) -> uint32_t {
            int h = n1, w = rs;
            asm volatile("" : "+s"(h), "+s"(w));
            const int ml = mo + w;
            sec = ml >= h;
            const int r = sec ? ml - h : ml;
            return (ml < rows_valid && col_ok) ? (uint32_t)((long)r * ldc + n) : OUT;
        };
        constexpr int PD = TM == 128 ? 1 : 2;         // passes of masters loaded ahead
        nf4 mb[PD + 1][8];
        auto prefetch = [&](int q, nf4* dst) {
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                bool sec;
                const uint32_t o = elem(q * 32 + it * 4, sec);
                dst[it] = __builtin_bit_cast(nf4, __builtin_amdgcn_raw_buffer_load_b128(
                    sec ? rm2 : rm1, o == OUT ? OUT : o * 4, 0, 2));
            }
        };
        if constexpr (EPI == EPI_SGD && TM == 256) {
            prefetch(0, mb[0]);
            prefetch(1, mb[1]);
        }

#ifdef MOE_GEMM_KT64
        if (nk > 0) {
            // Loads staged through registers.  rb holds the k-tile after the next: in the
            // slots of the first half of k-tile kt, vector q of k-tile kt+1 goes from rb[q] to
            // its LDS stage and rb[q] is reloaded with k-tile kt+2 (the LDS write reads rb[q]
            // when it issues), so each load has about one k-tile to arrive.  The barrier at
            // the end of k-tile kt publishes k-tile kt+1.  The vectors of a step are spread
            // over all its MFMA slots, so every wave layout (4, 8 or 16 slots) moves them all.
            nu4r rb[LPW];
            auto ldsoff = [&](int q, int kt) -> uint32_t {
                const uint32_t st = (uint32_t)(kt % NSt) * (STAGE * 2);
                const uint32_t o = (q < IPW_A) ? st + (uint32_t)(wave * IPW_A + q) * 1024u
                                               : st + TILE_A * 2 + (uint32_t)(wave * IPW_B + q - IPW_A) * 1024u;
                return o + (uint32_t)lane * 16u;
            };
            auto load = [&](int q, int kt) {
                if constexpr (GA == GA_ROWS) {
                    if (q < IPW_A) {
                        rb[q] = __builtin_bit_cast(nu4r, __builtin_amdgcn_raw_buffer_load_b128(
                            pa.r0, gvo[q], (uint32_t)(kt * BK) * 2u, 0));
                        return;
                    }
                }
                rb[q] = (q < IPW_A) ? load_one<AT, TM>(pa, q, kt * BK, wave)
                                    : load_one<BT>(pb, q - IPW_A, kt * BK, wave);
            };
            auto put = [&](int q, int kt) {
                *reinterpret_cast<nu4r*>(reinterpret_cast<char*>(lds) + ldsoff(q, kt)) = rb[q];
            };
#pragma unroll
            for (int q = 0; q < LPW; ++q) load(q, 0);
#pragma unroll
            for (int q = 0; q < LPW; ++q) { put(q, 0); load(q, 1); }
            __syncthreads();
            Frags fa, fb;
#pragma unroll
            for (int idx = 0; idx < NR; ++idx) read_one(lds, lds + TILE_A, 0, fa, idx);
            constexpr int HALF = KSTEPS / 2;
            static_assert(LPW % HALF == 0, "register-staged load parts");
            constexpr int PPS = LPW / HALF;                  // vectors moved per k-step
            for (int kt = 0; kt < nk; ++kt) {
                const int st = kt % NSt;
                const bf16* As = lds + st * STAGE;
                const bf16* Bs = lds + st * STAGE + TILE_A;
#pragma unroll
                for (int s = 0; s < KSTEPS; ++s) {
                    Frags& cur = (s & 1) ? fb : fa;
                    Frags& nxt = (s & 1) ? fa : fb;
                    if (s + 1 < KSTEPS) {
#pragma unroll
                        for (int i = 0; i < NMF; ++i) {
                            mfma_one(cur, i);
                            if (i < NR) read_one(As, Bs, s + 1, nxt, i);
                            if (s < HALF) {
#pragma unroll
                                for (int q = s * PPS + i * PPS / NMF; q < s * PPS + (i + 1) * PPS / NMF; ++q) {
                                    put(q, kt + 1);
                                    load(q, kt + 2);
                                }
                            }
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    } else {
                        // last step: publish k-tile kt+1, read its first fragments under the
                        // second half of the MFMAs
                        constexpr int h1 = NMF / 2;
#pragma unroll
                        for (int i = 0; i < h1; ++i) {
                            mfma_one(cur, i);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                        __syncthreads();
                        const int sn = (kt + 1) % NSt;
#pragma unroll
                        for (int i = h1; i < NMF; ++i) {
                            mfma_one(cur, i);
#pragma unroll
                            for (int idx = (i - h1) * NR / (NMF - h1); idx < (i - h1 + 1) * NR / (NMF - h1); ++idx)
                                read_one(lds + sn * STAGE, lds + sn * STAGE + TILE_A, 0, nxt, idx);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    }
                }
            }
        }
#else
        if (nk > 0) {
            if constexpr (KGATHER) {
#pragma unroll
                for (int t = 0; t <= DIST; ++t) idx_dma(t);
                wait_vm<0>();
            }
#pragma unroll
            for (int t = 0; t < DIST; ++t) {
                if constexpr (KGATHER) idx_read(t);
#pragma unroll
                for (int q = 0; q < LPW; ++q) dma(q, t);
            }
            if constexpr (KGATHER) idx_dma(DIST + 1);     // into k-tile 0's slot, now read
            wait_vm<LPW * (DIST - 1) + (KGATHER ? 1 : 0)>();
            __syncthreads();
            Frags fa, fb;
#pragma unroll
            for (int idx = 0; idx < NR; ++idx) read_one(lds, lds + TILE_A, 0, fa, idx);
            for (int kt = 0; kt < nk; ++kt) {
                const int st = kt % NSt;
                const bf16* As = lds + st * STAGE;
                const bf16* Bs = lds + st * STAGE + TILE_A;
                const int pf = kt + DIST;
                if constexpr (KGATHER) {
                    // the indices run two k-tiles ahead of the operand loads: k-tile pf + 2's go
                    // out now, are complete at the end of the next k-tile, and are read in the
                    // one after (three ring slots: pf being read, pf + 1 pending, pf + 2)
                    idx_dma(pf + 2);
                    idx_read(pf);
                }
#pragma unroll
                for (int s = 0; s < KSTEPS; ++s) {
                    Frags& cur = (s & 1) ? fb : fa;
                    Frags& nxt = (s & 1) ? fa : fb;
                    if (s + 1 < KSTEPS) {
                        // slot i: MFMA i, then fragment i of step s+1 and/or one load of k-tile pf
                        constexpr int lo = (NMF >= NR + PART) ? NR : NMF - PART;
#pragma unroll
                        for (int i = 0; i < NMF; ++i) {
                            mfma_one(cur, i);
                            if (i < NR) read_one(As, Bs, s + 1, nxt, i);
                            if (i >= lo && i - lo < PART) dma(s * PART + i - lo, pf);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    } else {
                        // last step: loads under the first half, then publish tile kt+1 and
                        // read its first fragments under the second half
                        constexpr int h1 = NMF / 2;
#pragma unroll
                        for (int i = 0; i < h1; ++i) {
                            mfma_one(cur, i);
#pragma unroll
                            for (int q = i * PART / h1; q < (i + 1) * PART / h1; ++q) dma(s * PART + q, pf);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                        wait_vm<LPW * (DIST - 1) + (KGATHER ? 1 : 0)>();
                        wait_lgkm0();
                        __syncthreads();
                        const int sn = (kt + 1) % NSt;
#pragma unroll
                        for (int i = h1; i < NMF; ++i) {
                            mfma_one(cur, i);
#pragma unroll
                            for (int idx = (i - h1) * NR / (NMF - h1); idx < (i - h1 + 1) * NR / (NMF - h1); ++idx)
                                read_one(lds + sn * STAGE, lds + sn * STAGE + TILE_A, 0, nxt, idx);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    }
                }
            }
            wait_vm<0>();
        }
#endif

        // ---- epilogue ------------------------------------------------------------------
        if constexpr (EPI == EPI_SGD) {
            // SGD step on the fp32 masters in place of storing the weight gradient.  The
            // tile goes out in 8 passes of 32 rows: the two wavefronts that own a pass's
            // rows put their accumulators in LDS (1 KB rows, 16-byte chunk c of row r at
            // c ^ r; two buffers, so one barrier per pass), then all 256 threads update
            // whole rows.  Each thread loads its masters two passes ahead into registers:
            // vector memory operations retire in issue order, so a wait for those loads
            // never covers the stores of the two passes before.
            static_assert(MODE == MODE_KSEG && OUT_F32 && NI == TM / 64 && NJ == 4,
                          "SGD epilogue: weight gradients, full wave layout");
            {
                float* stage = reinterpret_cast<float*>(lds);   // 2 x 32 rows x 1 KB
                constexpr int NP = TM / 32;                    // passes
                if constexpr (TM == 128) prefetch(0, mb[0]);
                __syncthreads();                               // every wave is past its last LDS read
#pragma unroll
                for (int q = 0; q < NP; ++q) {
                    if (q * 32 >= rows_valid) break;           // uniform
                    if (q + PD < NP) prefetch(q + PD, mb[(q + PD) % (PD + 1)]);
                    float* S = stage + (q & 1) * (32 * 256);
#pragma unroll
                    for (int i = 0; i < NI; ++i) {
                        if (rb + i * 32 != q * 32) continue;   // the waves that own rows q*32 ..
#pragma unroll
                        for (int j = 0; j < 4; ++j)
#pragma unroll
                            for (int g = 0; g < 4; ++g) {
                                const int c = (cb + j * 32 + g * 8 + hk * 4) >> 2;
                                *reinterpret_cast<nf4*>(S + rr * 256 + ((c ^ rr) << 2)) =
                                    nf4{acc[i][j][g * 4], acc[i][j][g * 4 + 1],
                                        acc[i][j][g * 4 + 2], acc[i][j][g * 4 + 3]};
                            }
                    }
                    __syncthreads();
#pragma unroll
                    for (int it = 0; it < 8; ++it) {
                        const int r = it * 4 + rs;
                        const nf4 gr = *reinterpret_cast<const nf4*>(S + r * 256 + ((qt ^ r) << 2));
                        bool sec;
                        const uint32_t o = elem(q * 32 + it * 4, sec);
                        const nf4 mv = mb[q % (PD + 1)][it];
                        nf4 w;
                        w.x = __builtin_fmaf(nlr, gr.x, mv.x);
                        w.y = __builtin_fmaf(nlr, gr.y, mv.y);
                        w.z = __builtin_fmaf(nlr, gr.z, mv.z);
                        w.w = __builtin_fmaf(nlr, gr.w, mv.w);
                        uint2 u;
                        bf16* h = reinterpret_cast<bf16*>(&u);
                        h[0] = (bf16)w.x; h[1] = (bf16)w.y; h[2] = (bf16)w.z; h[3] = (bf16)w.w;
                        const nu2 uv = {u.x, u.y};
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(nu4, w), sec ? rm2 : rm1,
                                                               o == OUT ? OUT : o * 4, 0, 2);
                        __builtin_amdgcn_raw_buffer_store_b64(uv, sec ? rw2 : rw1, o == OUT ? OUT : o * 2, 0, 2);
                    }
                }
            }
            return;
        }
        if constexpr (EPI == EPI_SCATTER) {
            // Router dX joined with the scatter: each token's dX is the sum of its k expert
            // rows of dXp (in pick order), then this tile's fp32 accumulator (dl Wg), then
            // the shared branch's part, in fp32, rounded once to bf16 -- the scatter kernel's
            // order, so dX is bitwise what router dX + scatter write.  The tile goes out in
            // two passes of 128 rows staged in LDS as fp32 (1 KB rows, 16-byte chunk q of
            // row r at q ^ (r & 63)); a thread then owns one 16-byte output vector (8
            // columns) of a row, and four rows' loads go out before their sums.
            static_assert(MODE == MODE_DENSE && !OUT_F32 && NI == 4 && NJ == 4, "scatter epilogue: router dX");
            constexpr int KS = MOE_SCATTER_FUSED_K;
            float* stage = reinterpret_cast<float*>(lds);
            int32_t* sslot = reinterpret_cast<int32_t*>(lds + NSt * STAGE + IDX_ELEMS);
            {   // thread r brings row r's slots (rows past the tile get slot 0: a valid row)
                nu4 s0 = {0u, 0u, 0u, 0u}, s1 = {0u, 0u, 0u, 0u};
                if (tid < rows_valid) {
                    const nu4* src = reinterpret_cast<const nu4*>(p.scat_slot + (long)(m0 + tid) * KS);
                    s0 = src[0]; s1 = src[1];
                }
                reinterpret_cast<nu4*>(sslot)[2 * tid] = s0;
                reinterpret_cast<nu4*>(sslot)[2 * tid + 1] = s1;
            }
            __syncthreads();                                   // every wave is past its last LDS read
            const int c = tid & 31;                            // the thread's output vector
            const bool col_ok = n0 + 8 * c < p.N;
            const long col = col_ok ? n0 + 8 * c : p.N - 8;    // loads stay inside the row
            const long ld = p.ldc;
            const rsrc_t rx = make_rsrc(reinterpret_cast<bf16*>(p.C) + (long)m0 * ld,
                                        ((long)(rows_valid - 1) * ld + p.N) * 2);
            const bf16* const rows = p.scat_rows;
            const bf16* const shared = p.scat_shared;
            auto body = [&](auto has_shared) {
                constexpr bool SH = decltype(has_shared)::value;
                for (int pass = 0; pass < 2; ++pass) {
                    if (pass * 128 >= rows_valid) break;       // uniform
#pragma unroll
                    for (int i = 0; i < NI; ++i) {
                        const int r = rb + i * 32 + rr - pass * 128;
                        if ((rb + i * 32) / 128 != pass) continue;   // wave-uniform
#pragma unroll
                        for (int j = 0; j < NJ; ++j)
#pragma unroll
                            for (int g = 0; g < 4; ++g) {
                                const int q = (cb + j * 32 + g * 8 + hk * 4) >> 2;
                                *reinterpret_cast<nf4*>(stage + r * 256 + ((q ^ (r & 63)) << 2)) =
                                    nf4{acc[i][j][g * 4], acc[i][j][g * 4 + 1], acc[i][j][g * 4 + 2],
                                        acc[i][j][g * 4 + 3]};
                            }
                    }
                    __syncthreads();
                    for (int it0 = 0; it0 < 16; it0 += 4) {
                        if (pass * 128 + it0 * 8 >= rows_valid) break;         // uniform
                        nu4 x[4][KS], xs[4];
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const int rt = pass * 128 + (it0 + u) * 8 + (tid >> 5);   // row in the tile
                            const nu4 sa = *reinterpret_cast<const nu4*>(sslot + rt * KS);
                            const nu4 sb = *reinterpret_cast<const nu4*>(sslot + rt * KS + 4);
#pragma unroll
                            for (int q = 0; q < KS; ++q) {
                                const uint32_t sl = q < 4 ? sa[q] : sb[q - 4];
                                x[u][q] = __builtin_nontemporal_load(
                                    reinterpret_cast<const nu4*>(rows + (long)sl * ld + col));
                            }
                            if constexpr (SH) {
                                const int rl = min(rt, rows_valid - 1);
                                xs[u] = __builtin_nontemporal_load(
                                    reinterpret_cast<const nu4*>(shared + (long)(m0 + rl) * ld + col));
                            }
                        }
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const int r = (it0 + u) * 8 + (tid >> 5);          // row in the pass
                            const int rt = pass * 128 + r;
                            float a8[8];
#pragma unroll
                            for (int v = 0; v < 8; ++v) a8[v] = 0.f;
#pragma unroll
                            for (int q = 0; q < KS; ++q) {
                                float f[8];
                                unpack8(x[u][q], f);
#pragma unroll
                                for (int v = 0; v < 8; ++v) a8[v] += f[v];
                            }
                            const nf4 g0 = *reinterpret_cast<const nf4*>(stage + r * 256 + (((2 * c) ^ (r & 63)) << 2));
                            const nf4 g1 = *reinterpret_cast<const nf4*>(stage + r * 256 + (((2 * c + 1) ^ (r & 63)) << 2));
                            a8[0] += g0.x; a8[1] += g0.y; a8[2] += g0.z; a8[3] += g0.w;
                            a8[4] += g1.x; a8[5] += g1.y; a8[6] += g1.z; a8[7] += g1.w;
                            if constexpr (SH) {
                                float f[8];
                                unpack8(xs[u], f);
#pragma unroll
                                for (int v = 0; v < 8; ++v) a8[v] += f[v];
                            }
                            const uint32_t o = (rt < rows_valid && col_ok) ? (uint32_t)(((long)rt * ld + n0 + 8 * c) * 2) : OUTB;
                            __builtin_amdgcn_raw_buffer_store_b128(pack8(a8), rx, o, 0, 0);
                        }
                    }
                    __syncthreads();                           // the pass's rows are read
                }
            };
            if (shared) body(std::true_type{});
            else body(std::false_type{});
            return;
        }
        if constexpr (EPI == EPI_STORE && OUT_F32) {
            // fp32 tile written out through LDS in two passes of 128 rows: each pass the
            // wavefronts that own those rows put their accumulators in LDS as 1 KB rows
            // (16-byte chunk q of row r at chunk q ^ (r & 63)), then all 256 threads store
            // whole rows
            float* stage = reinterpret_cast<float*>(lds);
            __syncthreads();                                   // every wave is past its last LDS read
            const int qt = tid & 63;
            const int npass = rows_valid > 128 ? 2 : 1;
            for (int pass = 0; pass < npass; ++pass) {
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    const int r = rb + i * 32 + rr - pass * 128;
                    if ((rb + i * 32) / 128 != pass) continue;   // wave-uniform
#pragma unroll
                    for (int j = 0; j < NJ; ++j)
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            const int q = (cb + j * 32 + g * 8 + hk * 4) >> 2;
                            *reinterpret_cast<float4*>(stage + r * 256 + ((q ^ (r & 63)) << 2)) =
                                make_float4(acc[i][j][g * 4], acc[i][j][g * 4 + 1], acc[i][j][g * 4 + 2],
                                            acc[i][j][g * 4 + 3]);
                        }
                }
                __syncthreads();
                // eight rows' LDS reads go out before their stores; every store is issued
                // unconditionally through a descriptor bounded to its output rows (weight
                // gradients: the two halves of the SGD epilogue's rm1 / rm2, chosen per row by
                // elem), so a row or column outside the tile gets an offset past the bound
                const rsrc_t rc = make_rsrc(reinterpret_cast<float*>(p.C) + (MODE == MODE_DENSE ? (long)e * p.ces : 0L) +
                                                ((MODE == MODE_ROWS) ? row_base + m0 : (long)m0) * p.ldc,
                                            ((long)(rows_valid - 1) * p.ldc + p.N) * 4);
                for (int it0 = 0; it0 < 32; it0 += 8) {
                    if (pass * 128 + it0 * 4 >= rows_valid) break;             // uniform
                    nf4 x[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const int r = (it0 + u) * 4 + wave;               // a wavefront stores whole rows
                        x[u] = *reinterpret_cast<const nf4*>(stage + r * 256 + ((qt ^ (r & 63)) << 2));
                    }
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        if constexpr (MODE == MODE_KSEG) {
                            bool sec;
                            const uint32_t o = elem(pass * 128 + (it0 + u) * 4, sec);
                            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(nu4, x[u]), sec ? rm2 : rm1,
                                                                   o == OUT ? OUT : o * 4, 0, 0);
                        } else {
                            const int ml = pass * 128 + (it0 + u) * 4 + wave;
                            const int n = n0 + qt * 4;
                            const uint32_t o = (ml < rows_valid && n < p.N) ? (uint32_t)(((long)ml * p.ldc + n) * 4) : OUT;
                            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(nu4, x[u]), rc, o, 0, 0);
                        }
                    }
                }
                __syncthreads();
            }
            return;
        }
        if constexpr ((EPI == EPI_STORE || EPI == EPI_STORE_BIAS || EPI == EPI_UP_SWIGLU ||
                       EPI == EPI_UP_SWIGLU_G) && !OUT_F32) {
            // bf16 tile written out through LDS: 512-byte rows of 32 chunks, chunk q of row r
            // at q ^ (r & 31); each lane puts its 4 consecutive columns (8 bytes) in place,
            // then the 256 threads store whole rows with 16-byte vectors
            bf16* stage = lds;
            __syncthreads();
            auto put = [&](int r, int c, const float* v) {      // c: first of 4 columns
                const int q = c >> 3;
                store4(stage + r * 256 + ((q ^ (r & 31)) << 3) + (c & 7), v);
            };
            // store the first ncols staged columns of the tile's rows: tile row r goes to
            // base + r ld, staged column c to column col_of(c) there (-1: nowhere).  One buffer
            // descriptor bounds the tile's rows, so every store is issued unconditionally (rows
            // past the tile fall outside it and are dropped), and the LDS reads of eight rows
            // go out before their stores instead of each store waiting for its own read.
            auto drain = [&](int ncols, bf16* base, long ld, auto col_of) {
                const int cpr = ncols / 8;                       // 16-byte chunks per row
                const int rows_per_it = 256 / cpr;
                const int q = tid % cpr;
                const int col = col_of(q * 8);
                const rsrc_t rd = make_rsrc(base, (long)rows_valid * ld * 2);
                const int nit = min(cpr, ((rows_valid + rows_per_it - 1) / rows_per_it + 7) & ~7);
                for (int i0 = 0; i0 < nit; i0 += 8) {
                    uint4 x[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const int r = (i0 + u) * rows_per_it + tid / cpr;
                        x[u] = *reinterpret_cast<const uint4*>(stage + r * 256 + ((q ^ (r & 31)) << 3));
                    }
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const int r = (i0 + u) * rows_per_it + tid / cpr;
                        const uint32_t off = col >= 0 ? (uint32_t)((r * ld + col) * 2) : OUTB;
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(nu4, x[u]), rd, off, 0, 0);
                    }
                }
            };
            if constexpr (EPI == EPI_STORE || EPI == EPI_STORE_BIAS) {
                // the bias (MLP down projection only) is added before the rounding to bf16
                constexpr int NB = EPI == EPI_STORE_BIAS ? NJ : 1;
                float bias[NB][4][4];
#pragma unroll
                for (int j = 0; j < NB; ++j)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int n = n0 + cb + j * 32 + g * 8 + hk * 4;
                        if (EPI == EPI_STORE_BIAS && n < p.N) load4(p.bias + (long)e * p.bias_es + n, bias[j][g]);
                        else bias[j][g][0] = bias[j][g][1] = bias[j][g][2] = bias[j][g][3] = 0.f;
                    }
#pragma unroll
                for (int i = 0; i < NI; ++i)
#pragma unroll
                    for (int j = 0; j < NJ; ++j)
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            float v[4];
#pragma unroll
                            for (int q = 0; q < 4; ++q)
                                v[q] = acc[i][j][g * 4 + q] + (EPI == EPI_STORE_BIAS ? bias[j < NB ? j : 0][g][q] : 0.f);
                            put(rb + i * 32 + rr, cb + j * 32 + g * 8 + hk * 4, v);
                        }
                __syncthreads();
                const long row0 = (MODE == MODE_ROWS) ? row_base + m0 : (long)m0;
                drain(256, reinterpret_cast<bf16*>(p.C) + row0 * p.ldc + n0, p.ldc,
                      [&](int c) { return n0 + c < p.N ? c : -1; });
            } else {
                // tile columns (B rows) alternate 32 W1 rows and the 32 W3 rows of the same
                // hidden units, so MFMA blocks j and j+1 (j even) pair H1 with H3.
                // Pass 1: [H1 | H3] staged as columns 0-127 | 128-255; pass 2: A in 0-127.
#pragma unroll
                for (int i = 0; i < NI; ++i)
#pragma unroll
                    for (int j = 0; j < NJ; j += 2)
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            float h1[4], h3[4];
#pragma unroll
                            for (int q = 0; q < 4; ++q) { h1[q] = acc[i][j][g * 4 + q]; h3[q] = acc[i][j + 1][g * 4 + q]; }
                            const int c = ((cb + j * 32) >> 6) * 32 + g * 8 + hk * 4;
                            put(rb + i * 32 + rr, c, h1);
                            put(rb + i * 32 + rr, 128 + c, h3);
                        }
                // EPI_UP_SWIGLU_G: the gates of this lane's accumulator rows, in flight while
                // the H rows drain
                float gsc[EPI == EPI_UP_SWIGLU_G ? NI : 1];
                if constexpr (EPI == EPI_UP_SWIGLU_G) {
#pragma unroll
                    for (int i = 0; i < NI; ++i) {
                        const int row = rb + i * 32 + rr;
                        gsc[i] = row < rows_valid ? p.row_scale[row_base + m0 + row] : 0.f;
                    }
                }
                __syncthreads();
                bf16* H = reinterpret_cast<bf16*>(p.C2);
                drain(256, H + (row_base + m0) * (2L * p.ffn) + hid0, 2L * p.ffn, [&](int c) {
                    const int hc = c & 127;
                    return hid0 + hc < p.ffn ? (c >= 128 ? p.ffn : 0) + hc : -1;
                });
                __syncthreads();
#pragma unroll
                for (int i = 0; i < NI; ++i)
#pragma unroll
                    for (int j = 0; j < NJ; j += 2)
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            float a[4];
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                a[q] = silu_fast_(acc[i][j][g * 4 + q]) * acc[i][j + 1][g * 4 + q];
                                if constexpr (EPI == EPI_UP_SWIGLU_G) a[q] *= gsc[i];
                            }
                            put(rb + i * 32 + rr, ((cb + j * 32) >> 6) * 32 + g * 8 + hk * 4, a);
                        }
                __syncthreads();
                drain(128, reinterpret_cast<bf16*>(p.C) + (row_base + m0) * (long)p.ffn + hid0, p.ffn,
                      [&](int c) { return hid0 + c < p.ffn ? c : -1; });
            }
            return;
        }
        if constexpr (EPI == EPI_DN_SWIGLU || EPI == EPI_DN_SWIGLU_G || EPI == EPI_DN_RELU ||
                      EPI == EPI_DN_GELU || EPI == EPI_UP_RELU || EPI == EPI_UP_GELU) {
            // Row-pass epilogue of the MLP forward (bias + activation: H and A out) and of the
            // activation backward (H in, dH out).  The fp32 accumulators go out in passes of
            // 32 rows through LDS (1 KB rows, 16-byte chunk c of row r at c ^ r, two buffers,
            // one barrier per pass); each thread then takes 8 consecutive columns of a row.
            // The forward loads its 8 biases once, before the passes; the backward reads H
            // (H1 and H3 for SwiGLU) as 16-byte vectors loaded two passes ahead.  Every load and
            // store inside the passes goes through a buffer descriptor bounded to the tile's
            // rows and is issued unconditionally (a lane outside the tile gets an offset past the
            // bound: its store is dropped, its load reads zeros), so the waits for H count
            // exactly and never cover the stores of the two passes before.
            // EPI_DN_SWIGLU_G: the accumulator is D = dY_t W2 for the row's token t, and
            // dA = g D with g the row's gate; each row's partial sum of D * silu(H1) * H3
            // over the tile's columns (its share of the gate gradient <dY_t, EO>) is added up
            // over the row's 32 threads in a fixed order and stored per N-tile.
            constexpr bool UP = EPI == EPI_UP_RELU || EPI == EPI_UP_GELU;
            constexpr bool GLU = EPI == EPI_DN_SWIGLU || EPI == EPI_DN_SWIGLU_G;
            constexpr bool GATED = EPI == EPI_DN_SWIGLU_G;
            constexpr int NH = GLU ? 2 : 1;                    // H vectors per 8 columns (backward)
            constexpr uint32_t OUT = 0x80000000u;              // past every bound
            float* stage = reinterpret_cast<float*>(lds);   // 2 x 32 rows x 1 KB
            const int c8 = tid & 31, rs = tid >> 5;            // 8-column chunk; row of an 8-row step
            const int n = n0 + c8 * 8;
            const bool col_ok = n < p.N;
            const long rowg = row_base + m0;                   // first row of the tile
            const int ldh = (int)p.ldh, ldc = (int)p.ldc, ffn = p.ffn;
            const int npass = (rows_valid + 31) >> 5;
            // backward: H in, dH out; forward: A out (C), H out (C2)
            const rsrc_t rh = make_rsrc(UP ? p.C2 : p.H + rowg * ldh,
                                        UP ? 0 : (long)rows_valid * ldh * 2);
            const rsrc_t rd = make_rsrc(reinterpret_cast<bf16*>(p.C) + rowg * ldc, (long)rows_valid * ldc * 2);
            const rsrc_t rh_out = make_rsrc(UP ? reinterpret_cast<bf16*>(p.C2) + rowg * ldc : p.C2,
                                            UP ? (long)rows_valid * ldc * 2 : 0);
            float bias8[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) bias8[k] = 0.f;
            if constexpr (UP) {
                if (col_ok) unpack8(*reinterpret_cast<const nu4*>(p.bias + (long)e * p.bias_es + n), bias8);
            }
            nu4 hb[3][4][NH];
            float gb[3][4];                                    // GATED: gates of the rows, same passes
            const rsrc_t rg = make_rsrc(GATED ? p.row_scale + rowg : nullptr, GATED ? (long)rows_valid * 4 : 0);
            const rsrc_t rdot = make_rsrc(GATED ? p.dot_part + (long)n_t * p.dot_ld + rowg : nullptr,
                                          GATED ? (long)rows_valid * 4 : 0);
            auto prefetch = [&](int q, int b) {
                if constexpr (!UP) {
#pragma unroll
                    for (int it = 0; it < 4; ++it) {
                        const int r = q * 32 + it * 8 + rs;
                        const bool ok = r < rows_valid && col_ok;
#pragma unroll
                        for (int h = 0; h < NH; ++h)
                            hb[b][it][h] = __builtin_bit_cast(nu4, __builtin_amdgcn_raw_buffer_load_b128(
                                rh, ok ? (uint32_t)(r * ldh + n + h * ffn) * 2 : OUT, 0, 0));
                        if constexpr (GATED)
                            gb[b][it] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                rg, r < rows_valid ? (uint32_t)r * 4 : OUT, 0, 0));
                    }
                }
            };
            prefetch(0, 0);
            if (npass > 1) prefetch(1, 1);
            __syncthreads();                                   // every wave is past its last LDS read
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                if (q >= npass) break;                         // uniform
                if (q + 2 < npass) prefetch(q + 2, (q + 2) % 3);
                float* S = stage + (q & 1) * (32 * 256);
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    if (rb + i * 32 != q * 32) continue;       // the waves that own rows q*32 ..
#pragma unroll
                    for (int j = 0; j < NJ; ++j)
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            const int c = (cb + j * 32 + g * 8 + hk * 4) >> 2;
                            *reinterpret_cast<nf4*>(S + rr * 256 + ((c ^ rr) << 2)) =
                                nf4{acc[i][j][g * 4], acc[i][j][g * 4 + 1], acc[i][j][g * 4 + 2],
                                    acc[i][j][g * 4 + 3]};
                        }
                }
                __syncthreads();
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const int r = it * 8 + rs;                 // row within the pass
                    const int rt = q * 32 + r;                 // row within the tile
                    const bool ok = rt < rows_valid && col_ok;
                    const nf4 x0 = *reinterpret_cast<const nf4*>(S + r * 256 + (((2 * c8) ^ r) << 2));
                    const nf4 x1 = *reinterpret_cast<const nf4*>(S + r * 256 + (((2 * c8 + 1) ^ r) << 2));
                    float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
                    const uint32_t o = ok ? (uint32_t)(rt * ldc + n) * 2 : OUT;
                    if constexpr (UP) {
                        float av[8];
#pragma unroll
                        for (int k = 0; k < 8; ++k) {
                            v[k] += bias8[k];
                            av[k] = (EPI == EPI_UP_RELU) ? fmaxf(v[k], 0.f) : gelu_fast_(v[k]);
                        }
                        __builtin_amdgcn_raw_buffer_store_b128(pack8(v), rh_out, o, 0, 0);
                        __builtin_amdgcn_raw_buffer_store_b128(pack8(av), rd, o, 0, 0);
                    } else {
                        float h1[8], o1[8];
                        unpack8(hb[q % 3][it][0], h1);
                        if constexpr (GLU) {
                            float h3[8], o3[8];
                            unpack8(hb[q % 3][it][NH - 1], h3);
                            if constexpr (GATED) {
                                float dot = 0.f;
#pragma unroll
                                for (int k = 0; k < 8; ++k) dot = fmaf(v[k], silu_fast_(h1[k]) * h3[k], dot);
                                dot = half_wave_sum(dot);              // this thread's row
                                const float g = gb[q % 3][it];
#pragma unroll
                                for (int k = 0; k < 8; ++k) v[k] *= g;
                                __builtin_amdgcn_raw_buffer_store_b32(
                                    __builtin_bit_cast(int, dot), rdot,
                                    (c8 == 0 && rt < rows_valid) ? (uint32_t)rt * 4 : OUT, 0, 0);
                            }
#pragma unroll
                            for (int k = 0; k < 8; ++k) {
                                o1[k] = v[k] * h3[k] * silu_grad_fast_(h1[k]);
                                o3[k] = v[k] * silu_fast_(h1[k]);
                            }
                            __builtin_amdgcn_raw_buffer_store_b128(pack8(o3), rd,
                                ok ? (uint32_t)(rt * ldc + n + ffn) * 2 : OUT, 0, 0);
                        } else {
#pragma unroll
                            for (int k = 0; k < 8; ++k)
                                o1[k] = v[k] * ((EPI == EPI_DN_RELU) ? (h1[k] > 0.f ? 1.f : 0.f) : gelu_grad_fast_(h1[k]));
                        }
                        __builtin_amdgcn_raw_buffer_store_b128(pack8(o1), rd, o, 0, 0);
                    }
                }
            }
            return;
        }
    };

    if constexpr (MODE == MODE_ROWS && TM == 128) {
        if (rows_valid <= 64) tile(Layout<2, 2>{});
        else tile(Layout<2, 4>{});
    } else if constexpr (MODE == MODE_ROWS) {
        if (rows_valid <= 64) tile(Layout<2, 2>{});
        else if (rows_valid <= 128) tile(Layout<4, 2>{});
        else tile(Layout<4, 4>{});
    } else {
        tile(Layout<TM / 64, 4>{});
    }
}

template <int MODE, bool AT, bool BT, int EPI, bool OUT_F32, int TM = 256, int GA = GA_NONE, bool PER = false>
__global__ void __launch_bounds__(NTHR, TM == 128 ? 2 : 1)
__attribute__((amdgpu_waves_per_eu(TM == 128 ? 2 : 1, TM == 128 ? 2 : 1)))
gemm_bf16_kernel(GemmParams p) {
    static_assert(!PER || MODE == MODE_KSEG, "persistent: weight gradients");
    __shared__ __attribute__((aligned(1024))) bf16 lds[TileLds<EPI, TM, GA>::ELEMS];
    const int tid = threadIdx.x;
    const int NT = p.paired ? (p.ffn + 127) / 128 : (p.N + BN - 1) / BN;

    int nreal;
    if (MODE == MODE_ROWS) nreal = p.tile_prefix[p.E] * NT;
    else if (MODE == MODE_KSEG) nreal = p.E * ((p.M + TM - 1) / TM) * NT;
    else nreal = ((p.M + BM - 1) / BM) * NT * (p.kchunk > 0 ? (p.K + p.kchunk - 1) / p.kchunk : 1);
    nreal = uni(nreal);
    // The persistent form (PER) takes its tiles from its XCD group's queue instead of its
    // block index: a grid of one workgroup per resident slot, each looping until the
    // group's tiles are handed out (an integer atomic per tile; which workgroup computes a
    // tile does not change its result).  Tickets walk the segments most rows first, so the
    // longest tiles go first and the short ones fill the tail.
    __shared__ int s_ticket;
    int L = blockIdx.x;
    int ticket = 0, per_total = 0, per_cg = 1, per_s0 = 0, per_tps = 1, per_g = 0;
    if constexpr (PER) {
        const int G = p.xcd_group, ng = 8 / G;
        per_g = uni((int)(blockIdx.x & 7) / G);
        per_tps = uni(nreal / p.E);
        per_s0 = (per_g * per_tps) / ng;
        per_cg = ((per_g + 1) * per_tps) / ng - per_s0;
        per_total = uni(p.E * per_cg);
        if (tid == 0) s_ticket = atomicAdd(p.queue + per_g, 1);
        __syncthreads();
        ticket = uni(s_ticket);
    } else {
        // Workgroups are dealt to the 8 XCDs round-robin by blockIdx. The XCDs form 8/G groups
        // of G; each group takes a contiguous, equal share of the tiles (of each segment's
        // tiles, for the weight gradients) and deals it round-robin to its members. G = 8 spreads neighbouring tiles over every L2 (each operand row is
        // fetched into all of them); G = 1 keeps them on one XCD (least fabric traffic, but the
        // requests of the co-resident tiles crowd one L2).
        const int G = p.xcd_group;
        const int x = L & 7, i = L >> 3, g = x / G, u = x - g * G, ng = 8 / G;
        const int li = i * G + u;
        if (MODE == MODE_KSEG) {
            // A weight-gradient tile costs in proportion to its segment's rows (K), so equal
            // tile counts per group are not equal work once the routing is skewed: every
            // group takes the same contiguous share of each segment's tiles instead.
            const int tps = uni(nreal / p.E);
            const int s0 = (g * tps) / ng, cg = ((g + 1) * tps) / ng - s0;
            if (cg == 0 || li >= p.E * cg) return;
            const int seg = li / cg;
            L = seg * tps + s0 + (li - seg * cg);
        } else {
            const int q = nreal / ng, r = nreal - q * ng;
            if (li >= q + (g < r ? 1 : 0)) return;
            L = g * q + min(g, r) + li;
        }
    }
    for (;;) {
        int next = 0;
        if constexpr (PER) {
            if (ticket >= per_total) break;                  // uniform: the group's tiles are all out
            const int seg = p.seg_order[ticket / per_cg];
            L = seg * per_tps + per_s0 + ticket % per_cg;
            if (tid == 0) next = atomicAdd(p.queue + per_g, 1);   // awaited after this tile
        }
        gemm_tile<MODE, AT, BT, EPI, OUT_F32, TM, GA>(p, L, lds);
        if constexpr (!PER) break;
        else {
            __syncthreads();                                 // the epilogue is done with LDS
            if (tid == 0) s_ticket = next;
            __syncthreads();
            ticket = uni(s_ticket);
        }
    }
}


// ---- host side -------------------------------------------------------------------------------
__global__ void __launch_bounds__(64) zero_queue_kernel(int32_t* q) {
    if (threadIdx.x < 8) q[threadIdx.x] = 0;
}

// Compute units of the current device (cached per device).
static int device_cus() {
    static int cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cus[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

template <int MODE, bool AT, bool BT, int EPI, bool OUT_F32, int TM = 256, int GA = GA_NONE, bool PER = false>
static hipError_t run(GemmParams p, int grid, hipStream_t s) {
    if (grid <= 0) return hipSuccess;
    if constexpr (PER) {
        // one workgroup per resident slot (two per CU with 128-row tiles), whole XCD rounds;
        // the queues start at zero
        if (p.xcd_group == 0) p.xcd_group = 8;
        if (p.xcd_group != 1 && p.xcd_group != 2 && p.xcd_group != 4 && p.xcd_group != 8) return hipErrorInvalidValue;
        if (!p.queue || !p.seg_order) return hipErrorInvalidValue;
        hipLaunchKernelGGL(zero_queue_kernel, dim3(1), dim3(64), 0, s, p.queue);
        const int slots = (device_cus() * (TM == 128 ? 2 : 1) + 7) & ~7;
        hipLaunchKernelGGL((gemm_bf16_kernel<MODE, AT, BT, EPI, OUT_F32, TM, GA, true>), dim3(slots),
                           dim3(NTHR), 0, s, p);
        return hipGetLastError();
    }
    // Whole XCD rounds; surplus workgroups exit at once. A multiple of 8 is a multiple of
    // every group count, so each group's slots cover its share of the tiles.
    if (p.xcd_group == 0) p.xcd_group = 8;
    if (p.xcd_group != 1 && p.xcd_group != 2 && p.xcd_group != 4 && p.xcd_group != 8) return hipErrorInvalidValue;
    if (MODE == MODE_KSEG) {
        // each of the 8/G groups needs slots for its share, ceil(tiles per segment / (8/G)),
        // of every segment
        const int ng = 8 / p.xcd_group;
        const long tps = (long)((p.M + TM - 1) / TM) * ((p.N + BN - 1) / BN);
        const long need = (long)ng * p.E * ((tps + ng - 1) / ng);
        if (need > 0x7ffffff0L) return hipErrorInvalidValue;
        grid = (int)need;
        if (grid <= 0) return hipSuccess;
    }
    grid = (grid + 7) & ~7;
    hipLaunchKernelGGL((gemm_bf16_kernel<MODE, AT, BT, EPI, OUT_F32, TM, GA>), dim3(grid), dim3(NTHR), 0, s, p);
    return hipGetLastError();
}

// Row tiles of 256 rows (one workgroup per CU), or of 128 (two per CU, short_rows()).
//
// 128-row tiles cost 1.5x the operand loads per flop of 256-row ones, but two workgroups share a
// CU, so one's prologue and epilogue run under the other's k-loop.  That pays only where a
// tile's fixed costs weigh most: a short K (at most 1024, 32 k-tiles) over few tiles (at most
// four rounds of 256-row tiles on the CUs).  Measured (T = 4096, d = 1024, E = 8, ffn = 4096,
// GELU): up projection 0.133 -> 0.111 ms, down dgrad 0.129 -> 0.104 ms; with K = 2048 or more
// tiles, or at T = 32768, they were 3-25% slower.  The SwiGLU activation-backward epilogue does
// not fit the halved register budget, so the rule covers the MLP kinds (bias + ReLU / GELU).
static bool short_rows(const ExpertGemmArgs& a, int K, int N) {
    if (a.expert == MOE_EXPERT_SWIGLU || K > 1024) return false;
    const long tiles = (long)((a.rows + BM - 1) / BM + a.E) * ((N + BN - 1) / BN);
    return tiles <= 4L * device_cus();
}

static GemmParams base_rows(const ExpertGemmArgs& a, int tm) {
    GemmParams p = {};
    p.E = a.E;
    p.offsets = a.offsets;
    p.tile_prefix = a.tile_prefix + (tm == 128 ? 1 : 2) * (MOE_MAX_EXPERTS + 1);    // 128- or 256-row tiles
    p.mtiles_ub = (a.rows + tm - 1) / tm + a.E;
    p.b2_kstart = -1;
    p.ffn = a.ffn;
    p.xcd_group = 4;     // measured: less fabric traffic than 8, steadier clock than 1 or 2
    return p;
}

template <int TM>
static hipError_t up_fwd_tm(const ExpertGemmArgs& a, hipStream_t s) {
    if (a.rows == 0) return hipSuccess;
    GemmParams p = base_rows(a, TM);
    p.A = (const bf16*)a.Xp; p.lda = a.d;
    p.B = (const bf16*)a.W1; p.ldb = a.d; p.bes = (long)a.ffn * a.d;
    p.K = a.d;
    if (a.expert == MOE_EXPERT_SWIGLU) {
        if constexpr (TM == 128) {
            return hipErrorInvalidValue;     // 128-row tiles: MLP kinds only
        } else {
            p.B2 = (const bf16*)a.W3; p.paired = 1; p.N = 2 * a.ffn;
            p.C = a.A; p.C2 = a.H;
            const int NT = (a.ffn + 127) / 128;
            if (a.token_of) {   // fused dispatch: rows of X through token_of, A gate-scaled
                p.A = (const bf16*)a.X; p.rows_tok = a.token_of; p.src_rows = a.T; p.row_scale = a.gate_of;
                return run<MODE_ROWS, false, false, EPI_UP_SWIGLU_G, false, TM, GA_ROWS>(p, p.mtiles_ub * NT, s);
            }
            return run<MODE_ROWS, false, false, EPI_UP_SWIGLU, false, TM>(p, p.mtiles_ub * NT, s);
        }
    }
    if (a.token_of) return hipErrorInvalidValue;      // fused dispatch: SwiGLU only
    p.N = a.ffn; p.C = a.A; p.C2 = a.H; p.ldc = a.ffn;
    p.bias = (const bf16*)a.b1; p.bias_es = a.ffn;
    const int NT = (a.ffn + BN - 1) / BN;
    if (a.expert == MOE_EXPERT_RELU)
        return run<MODE_ROWS, false, false, EPI_UP_RELU, false, TM>(p, p.mtiles_ub * NT, s);
    return run<MODE_ROWS, false, false, EPI_UP_GELU, false, TM>(p, p.mtiles_ub * NT, s);
}

#ifdef MOE_GEMM_KT64
hipError_t mfma_up_fwd(const ExpertGemmArgs& a, hipStream_t s) { return up_fwd_tm<256>(a, s); }
#else
hipError_t mfma_up_fwd(const ExpertGemmArgs& a, hipStream_t s) {
    return short_rows(a, a.d, a.ffn) ? up_fwd_tm<128>(a, s) : up_fwd_tm<256>(a, s);
}
bool mfma_up_fwd_short(const ExpertGemmArgs& a) { return short_rows(a, a.d, a.ffn); }
#endif

#ifndef MOE_GEMM_KT64     // the second build holds the up projection only
template <int TM>
static hipError_t down_fwd_tm(const ExpertGemmArgs& a, hipStream_t s) {
    if (a.rows == 0) return hipSuccess;
    GemmParams p = base_rows(a, TM);
    p.A = (const bf16*)a.A; p.lda = a.ffn;
    p.B = (const bf16*)a.W2; p.ldb = a.ffn; p.bes = (long)a.d * a.ffn;
    p.N = a.d; p.K = a.ffn;
    p.C = a.EO; p.ldc = a.d;
    const int NT = (a.d + BN - 1) / BN;
    if (a.b2) {
        p.bias = (const bf16*)a.b2; p.bias_es = a.d;
        return run<MODE_ROWS, false, false, EPI_STORE_BIAS, false, TM>(p, p.mtiles_ub * NT, s);
    }
    return run<MODE_ROWS, false, false, EPI_STORE, false, TM>(p, p.mtiles_ub * NT, s);
}

template <int TM>
static hipError_t down_dgrad_tm(const ExpertGemmArgs& a, hipStream_t s) {
    if (a.rows == 0) return hipSuccess;
    GemmParams p = base_rows(a, TM);
    const bool glu = a.expert == MOE_EXPERT_SWIGLU;
    const int hcols = glu ? 2 * a.ffn : a.ffn;
    p.A = (const bf16*)a.dEO; p.lda = a.d;
    p.B = (const bf16*)a.W2; p.ldb = a.ffn; p.bes = (long)a.d * a.ffn;   // B[k = c][n = j]
    p.N = a.ffn; p.K = a.d;
    p.C = a.dH; p.ldc = hcols;
    p.H = (const bf16*)a.H; p.ldh = hcols;
    const int grid = p.mtiles_ub * ((a.ffn + BN - 1) / BN);
    if constexpr (TM == 128) {  // 128-row tiles: MLP kinds only
        if (glu || a.token_of) return hipErrorInvalidValue;
        if (a.expert == MOE_EXPERT_RELU) return run<MODE_ROWS, false, true, EPI_DN_RELU, false, TM>(p, grid, s);
        return run<MODE_ROWS, false, true, EPI_DN_GELU, false, TM>(p, grid, s);
    } else {
        if (a.token_of) {       // fused dispatch: rows of dY through token_of, gate applied here
            if (!glu) return hipErrorInvalidValue;
            p.A = (const bf16*)a.dY; p.rows_tok = a.token_of; p.src_rows = a.T; p.row_scale = a.gate_of;
            p.dot_part = a.dgate_part; p.dot_ld = a.rows;
            return run<MODE_ROWS, false, true, EPI_DN_SWIGLU_G, false, TM, GA_ROWS>(p, grid, s);
        }
        if (glu) return run<MODE_ROWS, false, true, EPI_DN_SWIGLU, false, TM>(p, grid, s);
        if (a.expert == MOE_EXPERT_RELU) return run<MODE_ROWS, false, true, EPI_DN_RELU, false, TM>(p, grid, s);
        return run<MODE_ROWS, false, true, EPI_DN_GELU, false, TM>(p, grid, s);
    }
}
hipError_t mfma_down_fwd(const ExpertGemmArgs& a, hipStream_t s) { return down_fwd_tm<256>(a, s); }
hipError_t mfma_down_dgrad(const ExpertGemmArgs& a, hipStream_t s) {
    return short_rows(a, a.d, a.ffn) ? down_dgrad_tm<128>(a, s) : down_dgrad_tm<256>(a, s);
}

template <int TM>
static hipError_t up_dgrad_tm(const ExpertGemmArgs& a, hipStream_t s) {
    if (a.rows == 0) return hipSuccess;
    GemmParams p = base_rows(a, TM);
    const bool glu = a.expert == MOE_EXPERT_SWIGLU;
    const int hcols = glu ? 2 * a.ffn : a.ffn;
    p.A = (const bf16*)a.dH; p.lda = hcols;
    p.B = (const bf16*)a.W1; p.ldb = a.d; p.bes = (long)a.ffn * a.d;     // B[k = j][n = c]
    if (glu) { p.B2 = (const bf16*)a.W3; p.b2_kstart = a.ffn; }
    p.N = a.d; p.K = hcols;
    p.C = a.dXp; p.ldc = a.d;
    return run<MODE_ROWS, false, true, EPI_STORE, false, TM>(p, p.mtiles_ub * ((a.d + BN - 1) / BN), s);
}
hipError_t mfma_up_dgrad(const ExpertGemmArgs& a, hipStream_t s) { return up_dgrad_tm<256>(a, s); }

// With the SGD step in the epilogue, the weight gradients run persistent: one workgroup per
// CU takes its tiles from its XCD group's queue, segments with the most rows first (measured
// at T = 32768, E = 256: down 11.7 -> 11.25 ms, up 22.9 -> 22.0-22.5 ms against the block-
// index deal, with the up projection's 128-row tiles at two workgroups per CU).
hipError_t mfma_down_wgrad(const ExpertGemmArgs& a, hipStream_t s) {
    // dW2[e] (d x ffn) = dEO_e^T A_e: A operand = dEO as [k = row][m = c], B = A as [k][n = j]
    GemmParams p = {};
    p.E = a.E; p.offsets = a.offsets; p.b2_kstart = -1; p.ffn = a.ffn;
    p.queue = a.queue; p.seg_order = a.tile_prefix + 3 * (MOE_MAX_EXPERTS + 1);
    p.A = (const bf16*)a.dEO; p.lda = a.d;
    p.B = (const bf16*)a.A; p.ldb = a.ffn;
    p.M = a.d; p.N = a.ffn;
    p.C = a.dW2; p.ldc = a.ffn; p.ces = (long)a.d * a.ffn;
    const int grid = a.E * ((a.d + BM - 1) / BM) * ((a.ffn + BN - 1) / BN);
    p.xcd_group = 2;
    if (a.token_of) {           // fused dispatch: k-rows of dY through token_of; A is gate-scaled
        p.A = (const bf16*)a.dY; p.rows_tok = a.token_of; p.src_rows = a.T;
        if (a.W2m) {
            p.C = a.W2m; p.W = a.W2w; p.lr = a.lr;
            return run<MODE_KSEG, true, true, EPI_SGD, true, 256, GA_KA, true>(p, grid, s);
        }
        return run<MODE_KSEG, true, true, EPI_STORE, true, 256, GA_KA>(p, grid, s);
    }
    if (a.W2m) {    // SGD step on W2 in place of storing dW2
        p.C = a.W2m; p.W = a.W2w; p.lr = a.lr;
        return run<MODE_KSEG, true, true, EPI_SGD, true, 256, GA_NONE, true>(p, grid, s);
    }
    return run<MODE_KSEG, true, true, EPI_STORE, true>(p, grid, s);
}

hipError_t mfma_up_wgrad(const ExpertGemmArgs& a, hipStream_t s) {
    // [dW1 | dW3][e] (hcols x d) = dH_e^T Xp_e
    const bool glu = a.expert == MOE_EXPERT_SWIGLU;
    const int hcols = glu ? 2 * a.ffn : a.ffn;
    GemmParams p = {};
    p.E = a.E; p.offsets = a.offsets; p.b2_kstart = -1; p.ffn = a.ffn;
    p.queue = a.queue; p.seg_order = a.tile_prefix + 3 * (MOE_MAX_EXPERTS + 1);
    p.A = (const bf16*)a.dH; p.lda = hcols;
    p.B = (const bf16*)a.Xp; p.ldb = a.d;
    p.M = hcols; p.N = a.d;
    p.C = a.dW1; p.ldc = a.d; p.ces = (long)a.ffn * a.d;
    if (glu) { p.C2 = a.dW3; p.c2_mstart = a.ffn; }
    const int grid = a.E * ((hcols + BM - 1) / BM) * ((a.d + BN - 1) / BN);
    p.xcd_group = 2;
    if (a.token_of) {           // fused dispatch: k-rows of X through token_of
        p.B = (const bf16*)a.X; p.rows_tok = a.token_of; p.src_rows = a.T;
        if (a.W1m) {
            p.C = a.W1m; p.W = a.W1w; p.lr = a.lr;
            if (glu) { p.C2 = a.W3m; p.W2 = a.W3w; }
            return run<MODE_KSEG, true, true, EPI_SGD, true, 256, GA_KB, true>(p, grid, s);
        }
        return run<MODE_KSEG, true, true, EPI_STORE, true, 256, GA_KB>(p, grid, s);
    }
    if (a.W1m) {    // SGD step on W1 (and W3) in place of storing dW1 (dW3)
        p.C = a.W1m; p.W = a.W1w; p.lr = a.lr;
        if (glu) { p.C2 = a.W3m; p.W2 = a.W3w; }
        return run<MODE_KSEG, true, true, EPI_SGD, true, 256, GA_NONE, true>(p, grid, s);
    }
    return run<MODE_KSEG, true, true, EPI_STORE, true>(p, grid, s);
}

__global__ void __launch_bounds__(256) sum_partials_kernel(const float* part, float* out, long n4, int nsplit);

// K segments of the router logits: few output tiles (N = E <= 256 columns) would leave
// most CUs idle, so K = d is split until the tiles about fill the 256 CUs, keeping at
// least 256 columns (eight k-tiles) per segment and at most 8 segments.  Segment
// width is a multiple of 64 columns.
int router_logit_kchunk(int T, int E, int d) {
    const int tiles = ((T + BM - 1) / BM) * ((E + BN - 1) / BN);
    if (tiles <= 0) return 0;                         // no tokens: nothing to split
    int s = (256 + tiles - 1) / tiles;
    s = std::min(s, std::min(8, d / 256));
    if (s <= 1) return 0;
    return ((d + s - 1) / s + 63) / 64 * 64;
}
int router_logit_splits(int T, int E, int d) {
    const int kc = router_logit_kchunk(T, E, d);
    return kc > 0 ? (d + kc - 1) / kc : 1;
}

hipError_t mfma_router_logits(const RouterGemmArgs& a, hipStream_t s) {
    if (a.T == 0) return hipSuccess;
    GemmParams p = {};
    p.b2_kstart = -1;
    p.A = (const bf16*)a.X; p.lda = a.d;
    p.B = (const bf16*)a.Wg; p.ldb = a.d;
    p.M = a.T; p.N = a.E; p.K = a.d;
    p.C = a.logits; p.ldc = a.E;
    const int nseg = a.logit_part ? router_logit_splits(a.T, a.E, a.d) : 1;
    if (nseg > 1) {
        p.kchunk = router_logit_kchunk(a.T, a.E, a.d);
        p.C = a.logit_part; p.ces = (long)a.T * a.E;
    }
    const int grid = nseg * ((a.T + BM - 1) / BM) * ((a.E + BN - 1) / BN);
    hipError_t st = run<MODE_DENSE, false, false, EPI_STORE, true>(p, grid, s);
    if (st != hipSuccess || nseg == 1) return st;
    const long n4 = (long)a.T * a.E / 4;                 // E is a multiple of 8 on this path
    hipLaunchKernelGGL(sum_partials_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                       (const float*)a.logit_part, a.logits, n4, nseg);
    return hipGetLastError();
}

hipError_t mfma_router_dx(const RouterGemmArgs& a, hipStream_t s) {
    if (a.T == 0) return hipSuccess;
    GemmParams p = {};
    p.b2_kstart = -1;
    p.A = (const bf16*)a.dl; p.lda = a.E;
    p.B = (const bf16*)a.Wg; p.ldb = a.d;        // B[k = e][n = c]
    p.M = a.T; p.N = a.d; p.K = a.E;
    p.C = a.dXr; p.ldc = a.d;
    const int grid = ((a.T + BM - 1) / BM) * ((a.d + BN - 1) / BN);
    return run<MODE_DENSE, false, true, EPI_STORE, true>(p, grid, s);
}

hipError_t mfma_router_dx_scatter(const RouterGemmArgs& a, const ScatterArgs& sa, hipStream_t s) {
    if (a.T == 0) return hipSuccess;
    if (sa.k != MOE_SCATTER_FUSED_K || sa.T != a.T || a.d % 8 != 0) return hipErrorInvalidValue;
    GemmParams p = {};
    p.b2_kstart = -1;
    p.A = (const bf16*)a.dl; p.lda = a.E;
    p.B = (const bf16*)a.Wg; p.ldb = a.d;        // B[k = e][n = c]
    p.M = a.T; p.N = a.d; p.K = a.E;
    p.C = sa.dX; p.ldc = a.d;
    p.scat_rows = (const bf16*)sa.dXp; p.scat_slot = sa.slot_of; p.scat_shared = (const bf16*)sa.dXs;
    const int grid = ((a.T + BM - 1) / BM) * ((a.d + BN - 1) / BN);
    return run<MODE_DENSE, false, true, EPI_SCATTER, false>(p, grid, s);
}

// dWg (E x d) = dl^T X over K = T tokens.  With a partial buffer the T rows are
// split into nsplit chunks (KSEG segments without offsets) whose fp32 partial
// products are then summed in chunk order; without one, a single segment.
__global__ void __launch_bounds__(256) sum_partials_kernel(const float* part, float* out, long n4, int nsplit) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n4) return;
    float4 acc = reinterpret_cast<const float4*>(part)[i];
    for (int s = 1; s < nsplit; ++s) {
        const float4 v = reinterpret_cast<const float4*>(part)[(long)s * n4 + i];
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    reinterpret_cast<float4*>(out)[i] = acc;
}

// dWg's K = T is split into chunks of whole k-tiles until its E x d output tiles about fill
// the 256 CUs in one round (E = 8, d = 1024 gives 4 tiles: a single K = T tile each would leave
// the chip idle), keeping at least 128 rows (four k-tiles) a chunk and at most 64 chunks.
int router_dwg_kchunk(int T, int E, int d) {
    const int tiles = ((E + BM - 1) / BM) * ((d + BN - 1) / BN);
    int s = std::max(1, 256 / std::max(tiles, 1));
    s = std::min(s, std::min(64, T / 128));
    if (s <= 1) return 0;
    return ((T + s - 1) / s + BK - 1) / BK * BK;
}
int router_dwg_splits(int T, int E, int d) {
    const int kc = router_dwg_kchunk(T, E, d);
    return kc > 0 ? (T + kc - 1) / kc : 1;
}

hipError_t mfma_router_dwg(const RouterGemmArgs& a, hipStream_t s) {
    const int nsplit = a.dwg_part ? router_dwg_splits(a.T, a.E, a.d) : 1;
    GemmParams p = {};
    p.b2_kstart = -1;
    p.A = (const bf16*)a.dl; p.lda = a.E;
    p.B = (const bf16*)a.X; p.ldb = a.d;
    p.M = a.E; p.N = a.d; p.K = a.T;
    p.ldc = a.d;
    p.E = nsplit;
    if (nsplit > 1) {
        p.kchunk = router_dwg_kchunk(a.T, a.E, a.d);
        p.C = a.dwg_part; p.ces = (long)a.E * a.d;
    } else {
        p.C = a.dWg; p.ces = 0;
    }
    const int grid = nsplit * ((a.E + BM - 1) / BM) * ((a.d + BN - 1) / BN);
    hipError_t st = run<MODE_KSEG, true, true, EPI_STORE, true>(p, grid, s);
    if (st != hipSuccess || nsplit == 1) return st;
    const long n4 = (long)a.E * a.d / 4;
    hipLaunchKernelGGL(sum_partials_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                       (const float*)a.dwg_part, a.dWg, n4, nsplit);
    return hipGetLastError();
}

#endif  // MOE_GEMM_KT64
#ifdef MOE_GEMM_KT64
}  // namespace kt64
#endif
}  // namespace moe
