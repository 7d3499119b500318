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
//   * workgroup tile 256 x 256 x 64, 256 threads = 4 wavefronts in a 2 x 2
//     grid, each wavefront a 128 x 128 block of 4 x 4 MFMA 32x32x16 tiles with
//     fp32 accumulators;
//   * both operands sit in LDS K-contiguous ([rows][64] bf16, 128-byte rows of
//     eight 16-byte chunks, chunk XOR-swizzled by (row >> 1) & 7: the LDS has
//     64 four-byte banks, so the 16 lanes served together by a ds_read_b128
//     (16 consecutive rows, one chunk each) hit 16 distinct 16-byte bank
//     groups), double buffered (2 x 64 KB);
//   * every operand goes straight from global memory into LDS (buffer loads
//     with an LDS destination, bounds checked by the buffer descriptor so
//     ragged rows and k tails read as zero); K-contiguous operands are read
//     back with ds_read_b128, K-strided operands ([K][M] or [K][N] in memory,
//     kept in their natural layout) with the gfx950 transpose read
//     ds_read_b64_tr_b16, so the MFMA loop is the same for every layout;
//   * the MFMA is issued with the N operand first, so each lane's
//     accumulators hold 4 consecutive output columns: epilogue stores are
//     8-byte (bf16) or 16-byte (fp32) vectors;
//   * tiles are scheduled on the device from the expert offsets: ROWS mode
//     walks the m-tiles of every expert's row segment (prefix of per-expert
//     tile counts, binary search per workgroup); KSEG mode gives each expert
//     its own output and runs K over its row segment (empty segment -> the
//     output is written as zeros); DENSE is one plain GEMM.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int NTHR = 256;
constexpr int TILE_ELEMS = 256 * BK;            // one operand tile in LDS (bf16)
constexpr int GROUP_N = 8;                      // n-tiles per tile group (L2 reuse)

enum { MODE_ROWS = 0, MODE_KSEG = 1, MODE_DENSE = 2 };

typedef __amdgpu_buffer_rsrc_t rsrc_t;

struct GemmParams {
    // A operand (M x K).  AT = false: element (m, k) at A[m * lda + k];
    // AT = true: at A[k * lda + m].  m, k are absolute (segment offsets added).
    const bf16* A; long lda;
    // B operand (N x K).  BT = false: element (n, k) at B[e * bes + n * ldb + k];
    // BT = true: at B[e * bes + k * ldb + n].
    const bf16* B; const bf16* B2; long ldb; long bes;
    int b2_kstart;     // BT: rows k >= b2_kstart come from B2 at k - b2_kstart
    int paired;        // !BT: SwiGLU pairing, 128 hidden units per tile from B and B2
    int M, N, K, E;
    const int32_t* offsets;       // [E+1]
    const int32_t* tile_prefix;   // [E+1] m-tile prefix for BM-row tiles
    int mtiles_ub;                // upper bound of m-tiles (ROWS)
    // outputs
    void* C; void* C2; void* C3; long ldc; long ces;  // ces: per-expert stride (KSEG)
    int c2_mstart;     // KSEG: output rows m >= c2_mstart go to C2 at m - c2_mstart
    const bf16* bias; long bias_es;
    const bf16* H; long ldh; int ffn;
};

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Buffer resource over [base, base + bytes): loads past the end return zeros,
// which is how ragged rows, ragged k and column tails read as zero.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, long bytes) {
    if (bytes < 0) bytes = 0;
    if (bytes > 0x7fffffffL) bytes = 0x7fffffffL;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
typedef __attribute__((address_space(3))) void* lds_ptr_t;
__device__ __forceinline__ void bload_lds(rsrc_t r, const bf16* lds, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(lds), 16, voff, soff, 0, 0);
}

// ---- K-contiguous operand: straight from global memory into the LDS stage ----------
// One wave instruction fills 8 LDS rows (1 KB, lane l -> row l/8, physical chunk
// l%8); the lane therefore loads the logical chunk that the swizzle places at
// that physical chunk.  Wave w fills row blocks 8w .. 8w+7.
struct DirectOp {
    rsrc_t r0, r1;          // r1: second source of paired rows (W3)
    uint32_t ld_bytes;      // row pitch
    int paired;
};
__device__ __forceinline__ void issue_direct(const DirectOp& op, const bf16* stage, int k0) {
    const int lane = threadIdx.x & 63, wave = uni(threadIdx.x >> 6);
    // row 8j + l/8 has swizzle key ((8j + l/8) >> 1) & 7 = (4 (j & 1) + (l >> 4)) & 7
    const uint32_t row_off = (uint32_t)(lane >> 3) * op.ld_bytes;
    const uint32_t vo_even = row_off + ((uint32_t)((lane & 7) ^ (lane >> 4)) << 4);
    const uint32_t vo_odd = row_off + ((uint32_t)((lane & 7) ^ ((4 + (lane >> 4)) & 7)) << 4);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int j = wave * 8 + i;                       // row block: rows 8j .. 8j+7
        const uint32_t vo = (i & 1) ? vo_odd : vo_even;   // wave * 8 is even: j & 1 == i & 1
        int rowbase = 8 * j;
        rsrc_t r = op.r0;
        if (op.paired) {                                  // rows r: W1/W3 by (r >> 6) & 1
            rowbase = ((j >> 4) << 6) + ((8 * j) & 63);
            if ((j >> 3) & 1) r = op.r1;
        }
        bload_lds(r, stage + j * 512, vo, (uint32_t)rowbase * op.ld_bytes + (uint32_t)k0 * 2u);
    }
}

// ---- K-strided operand: natural [k][col] layout in LDS, transpose reads -------------
// Memory holds [k][col] with col contiguous.  A stage keeps 64 k-rows of 256
// columns (512-byte rows of 32 chunks), chunk XOR-swizzled by 2 * (row & 3).
// One wave instruction fills 2 rows (lane l -> row l/32, physical chunk l%32).
// Fragments come from ds_read_b64_tr_b16: inside each 16-lane group, lane l
// receives element (l & 3) of the 8-byte reads of lanes 4j + (l >> 2), j = 0..3.
// With lane 4j + m reading row k0 + j, columns c0 + 4m .. c0 + 4m + 3, lane l
// gets the four k values k0 .. k0 + 3 of column c0 + l: two reads give the eight
// consecutive k of one MFMA operand lane.  The swizzle keeps the four rows
// touched by one 16-lane group on 16 distinct bank pairs.
struct StridedOp {
    rsrc_t r0, r1;          // r1: rows k >= kswitch (W3 after W1 along k)
    uint32_t ld_bytes;
    int kswitch;
};
__device__ __forceinline__ void issue_strided(const StridedOp& op, const bf16* stage, int k0) {
    const int lane = threadIdx.x & 63, wave = uni(threadIdx.x >> 6);
    const uint32_t row_off = (uint32_t)(lane >> 5) * op.ld_bytes;
    const uint32_t vo_even = row_off + ((uint32_t)((lane & 31) ^ (2 * (lane >> 5))) << 4);
    const uint32_t vo_odd = row_off + ((uint32_t)((lane & 31) ^ (4 + 2 * (lane >> 5))) << 4);
    rsrc_t r = op.r0;
    int kk = k0;
    if (k0 >= op.kswitch) { r = op.r1; kk = k0 - op.kswitch; }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int j = wave * 8 + i;                       // rows 2j, 2j + 1 of the stage
        const uint32_t vo = (i & 1) ? vo_odd : vo_even;   // row & 3 = 2 (j & 1) + lane/32
        bload_lds(r, stage + j * 512, vo, (uint32_t)(kk + 2 * j) * op.ld_bytes);
    }
}

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s* lds_v4s_ptr;

// 32 columns [colbase, colbase + 32) x 16 k of k-step ks, in MFMA operand layout.
__device__ __forceinline__ bf16x8 read_strided(const bf16* T, int colbase, int ks) {
    const int lane = threadIdx.x & 63;
    const int L = lane & 15;
    const int col = colbase + 16 * ((lane >> 4) & 1) + 4 * (L & 3);
    const int pc = (col >> 3) ^ (2 * (L >> 2));           // k & 3 == L >> 2
    const int k = 16 * ks + 8 * (lane >> 5) + (L >> 2);
    const bf16* p0 = T + k * 256 + pc * 8 + (col & 7);
    const bf16* p1 = p0 + 4 * 256;                         // k + 4: same swizzle
    v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(p0));
    v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(p1));
    typedef short v8s __attribute__((ext_vector_type(8)));
    v8s v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// ---- MFMA fragments ----------------------------------------------------------------------
struct Frags { bf16x8 a[4], b[4]; };
__device__ __forceinline__ bf16x8 read_contig(const bf16* T, int rowbase, int ks) {
    const int lane = threadIdx.x & 63;
    const int rr = lane & 31, hk = lane >> 5;
    const int ch = ((2 * ks + hk) ^ ((rr >> 1) & 7)) << 3;
    return *reinterpret_cast<const bf16x8*>(T + (rowbase + rr) * BK + ch);
}
template <bool AT, bool BT>
__device__ __forceinline__ void read_frags(const bf16* As, const bf16* Bs, int ks, int wm, int wn, Frags& f) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
        f.a[i] = AT ? read_strided(As, wm * 128 + i * 32, ks) : read_contig(As, wm * 128 + i * 32, ks);
#pragma unroll
    for (int j = 0; j < 4; ++j)
        f.b[j] = BT ? read_strided(Bs, wn * 128 + j * 32, ks) : read_contig(Bs, wn * 128 + j * 32, ks);
}
__device__ __forceinline__ void mma(const Frags& f, f32x16 (&acc)[4][4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
}

// ---- epilogue helpers -----------------------------------------------------------------
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

// Grouped tile order inside an mt x nt tile grid: groups of GROUP_N n-tiles, all
// m-tiles of a group before the next group, so concurrently running tiles share
// A row blocks and B column blocks in L2.
__device__ __forceinline__ void grouped(int q, int mt, int nt, int& tm, int& tn) {
    const int gn = min(GROUP_N, nt);
    const int ng = q / (mt * gn);
    const int rem = q - ng * mt * gn;
    const int gsz = min(gn, nt - ng * gn);
    tm = rem / gsz;
    tn = ng * gn + (rem - tm * gsz);
}

// ---- the kernel ------------------------------------------------------------------------
template <int MODE, bool AT, bool BT, int EPI, bool OUT_F32>
__global__ void __launch_bounds__(NTHR, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_bf16_kernel(GemmParams p) {
    __shared__ __attribute__((aligned(1024))) bf16 lds[2][2][TILE_ELEMS];   // [stage][A/B]
    const int tid = threadIdx.x, lane = tid & 63, wave = uni(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    // ---- which tile: workgroups are dealt round-robin to the 8 XCDs, so give each
    // XCD a contiguous run of logical tiles (tiles that share operands meet in its L2)
    const int nwg = gridDim.x;
    int L = blockIdx.x;
    if ((nwg & 7) == 0) L = (L & 7) * (nwg >> 3) + (L >> 3);
    const int NT = p.paired ? (p.ffn + 127) / 128 : (p.N + BN - 1) / BN;
    int e = 0, m0 = 0, n_t = 0;
    long row_base = 0;        // absolute row of the segment start (ROWS) / K start (KSEG)
    int rows_valid = 0;       // valid rows of this tile in M
    int K = p.K;
    if (MODE == MODE_ROWS) {
        const int tmg = L / NT;
        if (tmg >= p.tile_prefix[p.E]) return;
        int lo = 0, hi = p.E;   // largest e with tile_prefix[e] <= tmg
        while (hi - lo > 1) {
            int mid = (lo + hi) >> 1;
            if (p.tile_prefix[mid] <= tmg) lo = mid; else hi = mid;
        }
        e = lo;
        const int mt = p.tile_prefix[e + 1] - p.tile_prefix[e];
        int tm;
        grouped(L - p.tile_prefix[e] * NT, mt, NT, tm, n_t);
        m0 = tm * BM;
        row_base = p.offsets[e];
        const int seg = p.offsets[e + 1] - p.offsets[e];
        rows_valid = min(BM, seg - m0);
    } else if (MODE == MODE_KSEG) {
        const int MT = (p.M + BM - 1) / BM;
        e = L / (MT * NT);
        if (e >= p.E) return;
        int tm;
        grouped(L - e * MT * NT, MT, NT, tm, n_t);
        m0 = tm * BM;
        rows_valid = min(BM, p.M - m0);
        if (p.offsets) {
            row_base = p.offsets[e];
            K = p.offsets[e + 1] - p.offsets[e];
        }
    } else {
        const int MT = (p.M + BM - 1) / BM;
        if (L >= MT * NT) return;
        int tm;
        grouped(L, MT, NT, tm, n_t);
        m0 = tm * BM;
        rows_valid = min(BM, p.M - m0);
    }
    e = uni(e); m0 = uni(m0); n_t = uni(n_t); rows_valid = uni(rows_valid); K = uni(K);
    row_base = (long)uni((int)row_base);
    const int n0 = n_t * BN;
    const int hid0 = n_t * 128;   // paired: first hidden unit of the tile
    const bf16* Be = p.B + (long)e * p.bes;
    const bf16* B2e = p.B2 ? p.B2 + (long)e * p.bes : nullptr;

    // ---- operand sources -----------------------------------------------------------------
    DirectOp da = {}, db = {};
    StridedOp sa = {}, sb = {};
    if (AT) {   // A[k][m]: k rows of the segment, columns m0 ..
        const bf16* base = p.A + row_base * p.lda + m0;
        sa.r0 = make_rsrc(base, ((long)K * p.lda - m0) * 2);
        sa.r1 = sa.r0;
        sa.ld_bytes = (uint32_t)(p.lda * 2);
        sa.kswitch = 0x7fffffff;
    } else {    // A[m][k]: rows m0 .. m0 + rows_valid of the segment
        const bf16* base = p.A + (row_base + m0) * p.lda;
        da.r0 = make_rsrc(base, (long)rows_valid * p.lda * 2);
        da.r1 = da.r0;
        da.ld_bytes = (uint32_t)(p.lda * 2);
        da.paired = 0;
    }
    if (BT) {   // B[k][n]
        if (MODE == MODE_KSEG) {
            const bf16* base = p.B + row_base * p.ldb + n0;
            sb.r0 = make_rsrc(base, ((long)K * p.ldb - n0) * 2);
            sb.r1 = sb.r0;
            sb.kswitch = 0x7fffffff;
        } else if (p.b2_kstart >= 0) {
            sb.r0 = make_rsrc(Be + n0, ((long)p.b2_kstart * p.ldb - n0) * 2);
            sb.r1 = make_rsrc(B2e + n0, ((long)(K - p.b2_kstart) * p.ldb - n0) * 2);
            sb.kswitch = p.b2_kstart;
        } else {
            sb.r0 = make_rsrc(Be + n0, ((long)K * p.ldb - n0) * 2);
            sb.r1 = sb.r0;
            sb.kswitch = 0x7fffffff;
        }
        sb.ld_bytes = (uint32_t)(p.ldb * 2);
    } else {    // B[n][k]
        if (p.paired) {
            db.r0 = make_rsrc(Be + (long)hid0 * p.ldb, (long)(p.ffn - hid0) * p.ldb * 2);
            db.r1 = make_rsrc(B2e + (long)hid0 * p.ldb, (long)(p.ffn - hid0) * p.ldb * 2);
            db.paired = 1;
        } else {
            db.r0 = make_rsrc(Be + (long)n0 * p.ldb, (long)min(BN, p.N - n0) * p.ldb * 2);
            db.r1 = db.r0;
            db.paired = 0;
        }
        db.ld_bytes = (uint32_t)(p.ldb * 2);
    }

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int nk = (K + BK - 1) / BK;
    // the loads of tile kt go straight into LDS stage st
    auto issue = [&](int kt, int st) {
        const int k0 = kt * BK;
        if (AT) issue_strided(sa, lds[st][0], k0); else issue_direct(da, lds[st][0], k0);
        if (BT) issue_strided(sb, lds[st][1], k0); else issue_direct(db, lds[st][1], k0);
    };

    if (nk > 0) {
        issue(0, 0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            const bool more = kt + 1 < nk;
            if (more) issue(kt + 1, cur ^ 1);
            const bf16* As = lds[cur][0];
            const bf16* Bs = lds[cur][1];
            // fragments of k-step s+1 are read while the MFMAs of k-step s run; the
            // scheduling fences keep the compiler from serialising reads and MFMAs
            Frags f0, f1;
            read_frags<AT, BT>(As, Bs, 0, wm, wn, f0);
            read_frags<AT, BT>(As, Bs, 1, wm, wn, f1);
            __builtin_amdgcn_sched_barrier(0);
            mma(f0, acc);
            __builtin_amdgcn_sched_barrier(0);
            read_frags<AT, BT>(As, Bs, 2, wm, wn, f0);
            __builtin_amdgcn_sched_barrier(0);
            mma(f1, acc);
            __builtin_amdgcn_sched_barrier(0);
            read_frags<AT, BT>(As, Bs, 3, wm, wn, f1);
            __builtin_amdgcn_sched_barrier(0);
            mma(f0, acc);
            __builtin_amdgcn_sched_barrier(0);
            mma(f1, acc);
            __builtin_amdgcn_sched_barrier(0);
            if (more) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }
    }

    // ---- epilogue ----------------------------------------------------------------------
    const int rr = lane & 31, hk = lane >> 5;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ml = wm * 128 + i * 32 + rr;       // local row
        if (ml >= rows_valid) continue;
        const long row = (MODE == MODE_ROWS) ? row_base + m0 + ml : (long)(m0 + ml);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float v[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) v[q] = acc[i][j][g * 4 + q];
                const int nl = wn * 128 + j * 32 + g * 8 + hk * 4;    // first of 4 local cols
                if (EPI == EPI_UP_SWIGLU) {
                    if (j >= 2) continue;
                    const int hid = hid0 + wn * 64 + j * 32 + g * 8 + hk * 4;
                    if (hid >= p.ffn) continue;
                    float h3[4], a[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        h3[q] = acc[i][j + 2][g * 4 + q];
                        a[q] = siluf_(v[q]) * h3[q];
                    }
                    bf16* H = reinterpret_cast<bf16*>(p.C2);
                    store4(H + row * (2L * p.ffn) + hid, v);
                    store4(H + row * (2L * p.ffn) + p.ffn + hid, h3);
                    store4(reinterpret_cast<bf16*>(p.C) + row * (long)p.ffn + hid, a);
                    continue;
                }
                const int n = n0 + nl;
                if (n >= p.N) continue;
                if (EPI == EPI_UP_RELU || EPI == EPI_UP_GELU) {
                    float b[4], a[4];
                    load4(p.bias + (long)e * p.bias_es + n, b);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        v[q] += b[q];
                        a[q] = (EPI == EPI_UP_RELU) ? fmaxf(v[q], 0.f) : geluf_(v[q]);
                    }
                    store4(reinterpret_cast<bf16*>(p.C2) + row * p.ldc + n, v);
                    store4(reinterpret_cast<bf16*>(p.C) + row * p.ldc + n, a);
                } else if (EPI == EPI_DN_SWIGLU) {
                    float h1[4], h3[4], d1[4], d3[4];
                    load4(p.H + row * p.ldh + n, h1);
                    load4(p.H + row * p.ldh + p.ffn + n, h3);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        d1[q] = v[q] * h3[q] * silu_gradf_(h1[q]);
                        d3[q] = v[q] * siluf_(h1[q]);
                    }
                    bf16* dH = reinterpret_cast<bf16*>(p.C);
                    store4(dH + row * p.ldc + n, d1);
                    store4(dH + row * p.ldc + p.ffn + n, d3);
                } else if (EPI == EPI_DN_RELU || EPI == EPI_DN_GELU) {
                    float h[4];
                    load4(p.H + row * p.ldh + n, h);
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        v[q] *= (EPI == EPI_DN_RELU) ? (h[q] > 0.f ? 1.f : 0.f) : gelu_gradf_(h[q]);
                    store4(reinterpret_cast<bf16*>(p.C) + row * p.ldc + n, v);
                } else {   // EPI_STORE
                    if (p.bias) {
                        float b[4];
                        load4(p.bias + (long)e * p.bias_es + n, b);
#pragma unroll
                        for (int q = 0; q < 4; ++q) v[q] += b[q];
                    }
                    if (MODE == MODE_KSEG) {
                        void* base = p.C;
                        long m = row;
                        if (p.C2 && m >= p.c2_mstart) { base = p.C2; m -= p.c2_mstart; }
                        store4(reinterpret_cast<float*>(base) + (long)e * p.ces + m * p.ldc + n, v);
                    } else if (OUT_F32) {
                        store4(reinterpret_cast<float*>(p.C) + row * p.ldc + n, v);
                    } else {
                        store4(reinterpret_cast<bf16*>(p.C) + row * p.ldc + n, v);
                    }
                }
            }
        }
    }
}

// ---- host side -------------------------------------------------------------------------------
template <int MODE, bool AT, bool BT, int EPI, bool OUT_F32>
static hipError_t run(const GemmParams& p, int grid, hipStream_t s) {
    if (grid <= 0) return hipSuccess;
    grid = (grid + 7) & ~7;   // whole XCD rounds; surplus workgroups exit at once
    hipLaunchKernelGGL((gemm_bf16_kernel<MODE, AT, BT, EPI, OUT_F32>), dim3(grid), dim3(NTHR), 0, s, p);
    return hipGetLastError();
}

static GemmParams base_rows(const ExpertGemmArgs& a) {
    GemmParams p = {};
    p.E = a.E;
    p.offsets = a.offsets;
    p.tile_prefix = a.tile_prefix + 2 * (MOE_MAX_EXPERTS + 1);    // 256-row tiles
    p.mtiles_ub = (a.rows + BM - 1) / BM + a.E;
    p.b2_kstart = -1;
    p.ffn = a.ffn;
    return p;
}

hipError_t mfma_up_fwd(const ExpertGemmArgs& a, hipStream_t s) {
    if (a.rows == 0) return hipSuccess;
    GemmParams p = base_rows(a);
    p.A = (const bf16*)a.Xp; p.lda = a.d;
    p.B = (const bf16*)a.W1; p.ldb = a.d; p.bes = (long)a.ffn * a.d;
    p.K = a.d;
    if (a.expert == MOE_EXPERT_SWIGLU) {
        p.B2 = (const bf16*)a.W3; p.paired = 1; p.N = 2 * a.ffn;
        p.C = a.A; p.C2 = a.H;
        const int NT = (a.ffn + 127) / 128;
        return run<MODE_ROWS, false, false, EPI_UP_SWIGLU, false>(p, p.mtiles_ub * NT, s);
    }
    p.N = a.ffn; p.C = a.A; p.C2 = a.H; p.ldc = a.ffn;
    p.bias = (const bf16*)a.b1; p.bias_es = a.ffn;
    const int NT = (a.ffn + BN - 1) / BN;
    if (a.expert == MOE_EXPERT_RELU)
        return run<MODE_ROWS, false, false, EPI_UP_RELU, false>(p, p.mtiles_ub * NT, s);
    return run<MODE_ROWS, false, false, EPI_UP_GELU, false>(p, p.mtiles_ub * NT, s);
}

hipError_t mfma_down_fwd(const ExpertGemmArgs& a, hipStream_t s) {
    if (a.rows == 0) return hipSuccess;
    GemmParams p = base_rows(a);
    p.A = (const bf16*)a.A; p.lda = a.ffn;
    p.B = (const bf16*)a.W2; p.ldb = a.ffn; p.bes = (long)a.d * a.ffn;
    p.N = a.d; p.K = a.ffn;
    p.C = a.EO; p.ldc = a.d;
    p.bias = (const bf16*)a.b2; p.bias_es = a.d;
    const int NT = (a.d + BN - 1) / BN;
    return run<MODE_ROWS, false, false, EPI_STORE, false>(p, p.mtiles_ub * NT, s);
}

hipError_t mfma_down_dgrad(const ExpertGemmArgs& a, hipStream_t s) {
    if (a.rows == 0) return hipSuccess;
    GemmParams p = base_rows(a);
    const bool glu = a.expert == MOE_EXPERT_SWIGLU;
    const int hcols = glu ? 2 * a.ffn : a.ffn;
    p.A = (const bf16*)a.dEO; p.lda = a.d;
    p.B = (const bf16*)a.W2; p.ldb = a.ffn; p.bes = (long)a.d * a.ffn;   // B[k = c][n = j]
    p.N = a.ffn; p.K = a.d;
    p.C = a.dH; p.ldc = hcols;
    p.H = (const bf16*)a.H; p.ldh = hcols;
    const int grid = p.mtiles_ub * ((a.ffn + BN - 1) / BN);
    if (glu) return run<MODE_ROWS, false, true, EPI_DN_SWIGLU, false>(p, grid, s);
    if (a.expert == MOE_EXPERT_RELU) return run<MODE_ROWS, false, true, EPI_DN_RELU, false>(p, grid, s);
    return run<MODE_ROWS, false, true, EPI_DN_GELU, false>(p, grid, s);
}

hipError_t mfma_up_dgrad(const ExpertGemmArgs& a, hipStream_t s) {
    if (a.rows == 0) return hipSuccess;
    GemmParams p = base_rows(a);
    const bool glu = a.expert == MOE_EXPERT_SWIGLU;
    const int hcols = glu ? 2 * a.ffn : a.ffn;
    p.A = (const bf16*)a.dH; p.lda = hcols;
    p.B = (const bf16*)a.W1; p.ldb = a.d; p.bes = (long)a.ffn * a.d;     // B[k = j][n = c]
    if (glu) { p.B2 = (const bf16*)a.W3; p.b2_kstart = a.ffn; }
    p.N = a.d; p.K = hcols;
    p.C = a.dXp; p.ldc = a.d;
    return run<MODE_ROWS, false, true, EPI_STORE, false>(p, p.mtiles_ub * ((a.d + BN - 1) / BN), s);
}

hipError_t mfma_down_wgrad(const ExpertGemmArgs& a, hipStream_t s) {
    // dW2[e] (d x ffn) = dEO_e^T A_e: A operand = dEO as [k = row][m = c], B = A as [k][n = j]
    GemmParams p = {};
    p.E = a.E; p.offsets = a.offsets; p.b2_kstart = -1; p.ffn = a.ffn;
    p.A = (const bf16*)a.dEO; p.lda = a.d;
    p.B = (const bf16*)a.A; p.ldb = a.ffn;
    p.M = a.d; p.N = a.ffn;
    p.C = a.dW2; p.ldc = a.ffn; p.ces = (long)a.d * a.ffn;
    const int grid = a.E * ((a.d + BM - 1) / BM) * ((a.ffn + BN - 1) / BN);
    return run<MODE_KSEG, true, true, EPI_STORE, true>(p, grid, s);
}

hipError_t mfma_up_wgrad(const ExpertGemmArgs& a, hipStream_t s) {
    // [dW1 | dW3][e] (hcols x d) = dH_e^T Xp_e
    const bool glu = a.expert == MOE_EXPERT_SWIGLU;
    const int hcols = glu ? 2 * a.ffn : a.ffn;
    GemmParams p = {};
    p.E = a.E; p.offsets = a.offsets; p.b2_kstart = -1; p.ffn = a.ffn;
    p.A = (const bf16*)a.dH; p.lda = hcols;
    p.B = (const bf16*)a.Xp; p.ldb = a.d;
    p.M = hcols; p.N = a.d;
    p.C = a.dW1; p.ldc = a.d; p.ces = (long)a.ffn * a.d;
    if (glu) { p.C2 = a.dW3; p.c2_mstart = a.ffn; }
    const int grid = a.E * ((hcols + BM - 1) / BM) * ((a.d + BN - 1) / BN);
    return run<MODE_KSEG, true, true, EPI_STORE, true>(p, grid, s);
}

hipError_t mfma_router_logits(const RouterGemmArgs& a, hipStream_t s) {
    if (a.T == 0) return hipSuccess;
    GemmParams p = {};
    p.b2_kstart = -1;
    p.A = (const bf16*)a.X; p.lda = a.d;
    p.B = (const bf16*)a.Wg; p.ldb = a.d;
    p.M = a.T; p.N = a.E; p.K = a.d;
    p.C = a.logits; p.ldc = a.E;
    const int grid = ((a.T + BM - 1) / BM) * ((a.E + BN - 1) / BN);
    return run<MODE_DENSE, false, false, EPI_STORE, true>(p, grid, s);
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

hipError_t mfma_router_dwg(const RouterGemmArgs& a, hipStream_t s) {
    // dWg (E x d) = dl^T X: one K segment [0, T)
    GemmParams p = {};
    p.E = 1; p.offsets = nullptr; p.K = a.T; p.b2_kstart = -1;
    p.A = (const bf16*)a.dl; p.lda = a.E;
    p.B = (const bf16*)a.X; p.ldb = a.d;
    p.M = a.E; p.N = a.d;
    p.C = a.dWg; p.ldc = a.d; p.ces = 0;
    const int grid = ((a.E + BM - 1) / BM) * ((a.d + BN - 1) / BN);
    return run<MODE_KSEG, true, true, EPI_STORE, true>(p, grid, s);
}

}  // namespace moe
