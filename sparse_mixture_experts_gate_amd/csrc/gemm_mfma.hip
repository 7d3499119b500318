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
//   * both operands sit in LDS K-contiguous ([rows][64] bf16, 16-byte chunks
//     XOR-swizzled by row & 7 so that the 8 lanes of a ds_read_b128 phase hit
//     8 distinct bank groups), double buffered (2 x 64 KB);
//   * K-contiguous operands are copied global -> registers -> LDS with
//     16-byte loads; K-strided operands ([K][M] or [K][N] in memory) are
//     loaded as 8 x 8 blocks and transposed in registers on the way, so the
//     MFMA loop is the same for every layout;
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

enum { MODE_ROWS = 0, MODE_KSEG = 1, MODE_DENSE = 2 };

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

// ---- global -> register -> LDS movers ----------------------------------------

// K-contiguous tile: 256 rows x 64 k.  Thread owns chunk c = tid & 7 of rows
// r0 + 32 i.  Row pointers come from a callable (segment / pairing aware).
struct KContig {
    uint4 v[8];
    template <class RowPtr>
    __device__ __forceinline__ void load(RowPtr rowptr, int k0, int k_valid) {
        const int c = threadIdx.x & 7, r0 = threadIdx.x >> 3;
        const bool kin = c * 8 < k_valid;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const bf16* p = rowptr(r0 + 32 * i);
            v[i] = (kin && p) ? *reinterpret_cast<const uint4*>(p + k0 + c * 8) : make_uint4(0, 0, 0, 0);
        }
    }
    __device__ __forceinline__ void store(bf16* lds) const {
        const int c = threadIdx.x & 7, r0 = threadIdx.x >> 3;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = r0 + 32 * i;
            *reinterpret_cast<uint4*>(lds + r * BK + ((c ^ (r & 7)) << 3)) = v[i];
        }
    }
};

__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

// K-strided tile: 64 k-rows x 256 columns in memory ([k][col], col contiguous).
// Thread owns the 8 x 8 block (k-block kb = tid & 7, column block mb = tid >> 3)
// and transposes it so LDS again holds [col][k].
struct KStrided {
    uint4 v[8];
    __device__ __forceinline__ void load(const bf16* base, long ld, int k_valid, int col_valid) {
        const int kb = threadIdx.x & 7, mb = threadIdx.x >> 3;
        const bool cin = mb * 8 < col_valid;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int k = kb * 8 + r;
            v[r] = (cin && k < k_valid) ? *reinterpret_cast<const uint4*>(base + (long)k * ld + mb * 8)
                                        : make_uint4(0, 0, 0, 0);
        }
    }
    __device__ __forceinline__ void store(bf16* lds) const {
        const int kb = threadIdx.x & 7, mb = threadIdx.x >> 3;
        const uint32_t* w = reinterpret_cast<const uint32_t*>(v);   // w[4 r + c/2]
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            uint4 o;
            const int q = c >> 1;
            if ((c & 1) == 0) {
                o.x = lo_pair(w[0 * 4 + q], w[1 * 4 + q]);
                o.y = lo_pair(w[2 * 4 + q], w[3 * 4 + q]);
                o.z = lo_pair(w[4 * 4 + q], w[5 * 4 + q]);
                o.w = lo_pair(w[6 * 4 + q], w[7 * 4 + q]);
            } else {
                o.x = hi_pair(w[0 * 4 + q], w[1 * 4 + q]);
                o.y = hi_pair(w[2 * 4 + q], w[3 * 4 + q]);
                o.z = hi_pair(w[4 * 4 + q], w[5 * 4 + q]);
                o.w = hi_pair(w[6 * 4 + q], w[7 * 4 + q]);
            }
            const int r = mb * 8 + c;
            *reinterpret_cast<uint4*>(lds + r * BK + ((kb ^ c) << 3)) = o;
        }
    }
};

// ---- MFMA on one LDS stage -------------------------------------------------------
__device__ __forceinline__ void mma_stage(const bf16* As, const bf16* Bs, f32x16 (&acc)[4][4],
                                          int wm, int wn) {
    const int lane = threadIdx.x & 63;
    const int rr = lane & 31, hk = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
        const int ch = ((2 * ks + hk) ^ (rr & 7)) << 3;
        bf16x8 af[4], bfr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            af[i] = *reinterpret_cast<const bf16x8*>(As + (wm * 128 + i * 32 + rr) * BK + ch);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            bfr[j] = *reinterpret_cast<const bf16x8*>(Bs + (wn * 128 + j * 32 + rr) * BK + ch);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
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

// ---- the kernel ------------------------------------------------------------------------
template <int MODE, bool AT, bool BT, int EPI, bool OUT_F32>
__global__ void __launch_bounds__(NTHR, 1) gemm_bf16_kernel(GemmParams p) {
    __shared__ __attribute__((aligned(16))) bf16 lds[2][2][TILE_ELEMS];   // [stage][A/B]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // ---- which tile -----------------------------------------------------------
    const int NT = p.paired ? (p.ffn + 127) / 128 : (p.N + BN - 1) / BN;
    int e = 0, m0 = 0, n_t = 0;
    long row_base = 0;        // absolute row of the segment start (ROWS) / K start (KSEG)
    int rows_valid = 0;       // valid rows of this tile in M
    int K = p.K;
    const int L = blockIdx.x;
    if (MODE == MODE_ROWS) {
        const int tm = L / NT;
        n_t = L - tm * NT;
        if (tm >= p.tile_prefix[p.E]) return;
        int lo = 0, hi = p.E;   // largest e with tile_prefix[e] <= tm
        while (hi - lo > 1) {
            int mid = (lo + hi) >> 1;
            if (p.tile_prefix[mid] <= tm) lo = mid; else hi = mid;
        }
        e = lo;
        m0 = (tm - p.tile_prefix[e]) * BM;
        row_base = p.offsets[e];
        const int seg = p.offsets[e + 1] - p.offsets[e];
        rows_valid = min(BM, seg - m0);
    } else if (MODE == MODE_KSEG) {
        const int MT = (p.M + BM - 1) / BM;
        e = L / (MT * NT);
        const int rem = L - e * MT * NT;
        const int tm = rem / NT;
        n_t = rem - tm * NT;
        m0 = tm * BM;
        rows_valid = min(BM, p.M - m0);
        if (p.offsets) {
            row_base = p.offsets[e];
            K = p.offsets[e + 1] - p.offsets[e];
        }
    } else {
        const int tm = L / NT;
        n_t = L - tm * NT;
        m0 = tm * BM;
        rows_valid = min(BM, p.M - m0);
    }
    const int n0 = n_t * BN;
    const bf16* Be = p.B + (long)e * p.bes;
    const bf16* B2e = p.B2 ? p.B2 + (long)e * p.bes : nullptr;
    const int hid0 = n_t * 128;   // paired: first hidden unit of the tile

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // operand row pointers (K-contiguous cases)
    auto a_row = [&](int r) -> const bf16* {
        const int rr = min(r, rows_valid - 1);
        return p.A + (row_base + m0 + rr) * p.lda;
    };
    auto b_row = [&](int r) -> const bf16* {
        if (p.paired) {
            const int hid = hid0 + (r >> 7) * 64 + (r & 63);
            const int h = min(hid, p.ffn - 1);
            return (((r >> 6) & 1) ? B2e : Be) + (long)h * p.ldb;
        }
        const int n = min(n0 + r, p.N - 1);
        return Be + (long)n * p.ldb;
    };

    KContig ga, gb;
    KStrided ta, tb;
    const int nk = (K + BK - 1) / BK;

    auto load_tile = [&](int kt) {
        const int k0 = kt * BK;
        const int kv = K - k0;
        if (AT) {
            // A[k][m]: rows k = row_base + k0 .., columns m0 ..
            ta.load(p.A + (row_base + k0) * p.lda + m0, p.lda, kv, rows_valid);
        } else {
            ga.load(a_row, k0, kv);
        }
        if (BT) {
            const bf16* bb = Be;
            int kk = k0;
            if (p.b2_kstart >= 0 && k0 >= p.b2_kstart) { bb = B2e; kk = k0 - p.b2_kstart; }
            if (MODE == MODE_KSEG) bb = p.B + row_base * p.ldb;     // B[k][n] rows of the segment
            tb.load(bb + (long)kk * p.ldb + n0, p.ldb, kv, p.N - n0);
        } else {
            gb.load(b_row, k0, kv);
        }
    };
    auto store_tile = [&](int stage) {
        if (AT) ta.store(lds[stage][0]); else ga.store(lds[stage][0]);
        if (BT) tb.store(lds[stage][1]); else gb.store(lds[stage][1]);
    };

    if (nk > 0) {
        load_tile(0);
        store_tile(0);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            if (kt + 1 < nk) load_tile(kt + 1);
            mma_stage(lds[cur][0], lds[cur][1], acc, wm, wn);
            if (kt + 1 < nk) store_tile(cur ^ 1);
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
