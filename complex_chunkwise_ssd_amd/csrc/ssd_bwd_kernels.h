// ssd_bwd_kernels.h -- gfx950 kernels of the backward of the complex chunkwise
// SSD scan: the gradients that the "Extending" guide (Path B Step 3, the
// autograd Function of a scan kernel) asks for -- true upstream gradients for
// y and final_state, a gradient for every input (x, A, B_t, C_t, dt and the
// initial state). A complex input z receives dl/dRe(z) + i dl/dIm(z).
//
// Per (b, h) and chunk c of Q tokens (running sums Lam inside the chunk,
// L[l,s] = exp(Lam[l] - Lam[s]) on l >= s, e_in = exp(Lam),
// e_end = exp(Lam[Q-1] - Lam)), with H the state entering the chunk and G the
// adjoint of the state leaving it, written without conjugation:
//   M = (C B^T) o L,   V = (gy x^T) o L
//   conj(gx) = M^T gy + diag(e_end) B G
//   conj(gB) = V^T C  + diag(e_end) x G^T
//   conj(gC) = V B    + diag(e_in) gy H^T
// and the gradient of a_t = softplus(dt_t) A collects, for every pair of
// tokens l >= s whose decay exp(Lam_l - Lam_s) spans t, that pair's share of
// the loss: with O/I the output/input-side row sums of the pairs inside the
// chunk and Off/In those of the pairs that cross its edges,
//   dF/da_t = sum_{j>=t} (O_j - I_j + Off_j) + sum_{s<t} In_s + exp(Lam[Q-1]) <H, G>
//   O_l = C_l . (V B)_l,  I_s = B_s . (V^T C)_s,
//   Off_l = C_l . (e_in gy H^T)_l,  In_s = B_s . (e_end x G^T)_s
//   ga = conj(dF/da),  gdt = Re(conj(A) ga) sigmoid(dt),  gA = sum softplus(dt) ga.
// G moves left by G <- exp(Lam[Q-1]) G + (diag(e_in) C)^T gy, H right by the
// forward's H <- exp(Lam[Q-1]) H + (diag(e_end) B)^T x.
//
// Three launches: bwd_state_kernel<R, false> writes every chunk's entering
// state H, bwd_state_kernel<R, true> every chunk's leaving adjoint G (and the
// initial-state gradient), then bwd_chunk_kernel<R> evaluates all chunks in
// parallel from those; bwd_reduce_gA_kernel sums the per-chunk shares of gA
// in a fixed order. Every contraction is a real-split fp32 MFMA 16x16x4 with
// operands from LDS planes; running sums of a are taken in double.
//
// N or D above 64: the state is cut into 64 x 64 blocks (n-slice S, d-slice T).
// A block's state and adjoint evolve on their own (B[:, S] and x[:, T] only),
// and every gradient is a sum over slices of the same expressions on the
// slices' columns: gx[:, T] = sum_S (M_S^T gy_T + e_end B_S G_ST) with M_S the
// Gram of the n-slice, gB[:, S] and gC[:, S] sum over T, and dF/da -- whose row
// sums are products of an n-sum and a d-sum -- over all pairs (S, T). So each
// (sequence, S, T) is a "virtual sequence" of the passes above, the chunk pass
// writes partial gradients per slice, and bwd_slice_sum_kernel adds them in a
// fixed order into the output layout.
#pragma once

#include <ssd_kernels.h>

namespace ssd {

constexpr int kBwdMaxRows = 32;  // tokens the backward evaluates per chunk, at most
constexpr int kBwdLd = 81;       // row stride (floats) of the chunk pass's [row][64] planes
constexpr int kStLd = 65;        // ... of its 64 x 64 state planes
constexpr int kStrideA = 80;     // ... of the state pass's [row][64] planes
constexpr int kStateFloats = 64 * 64 * 2;  // one padded complex 64 x 64 state
constexpr int kDecayWave = 3;   // chunk pass: the running sums of a chunk (no Gram tile)
constexpr int kGradWave = 7;    // ... the previous chunk's decay gradients
constexpr int kBwdGroups = 256;  // workgroups of the chunk pass: one per compute unit
constexpr uint32_t kBwdOut = 0x80000000u;  // a byte offset past every buffer

struct BwdParams {
    const float *x;         // (B, T, H, D) complex
    const float *A;         // (H) complex
    const float *Bt;        // (B, T, H, N) complex
    const float *Ct;        // (B, T, H, N) complex
    const float *dt;        // (B, T, H)
    const float *init;      // (B, H, N, D) complex or null
    const float *gy;        // (B, T, H, D)
    const float *gfinal;    // (B, H, N, D) complex or null
    float *gx;              // (B, T, H, D) complex
    float *gA;              // (H) complex
    float *gB;              // (B, T, H, N) complex
    float *gC;              // (B, T, H, N) complex
    float *gdt;             // (B, T, H)
    float *ginit;           // (B, H, N, D) complex or null
    float *fwd_states;      // (B, H, nc, 64, 64) complex: state entering each chunk
    float *adj_states;      // (B, H, nc, 64, 64) complex: adjoint leaving each chunk, conjugated
    float *gA_part;         // (B, H, ns, nc) complex: each chunk's (and slice's) share of gA
    int B, T, H, N, D, Q, nc;
    // State slices: nnb x ndb blocks of 64 x 64 (ns = nnb * ndb); with ns > 1 the
    // chunk pass writes partial gradients, complex (or real for dt) in the
    // (B, T, H, width) layout: gx_part (nnb, ..., D), gB_part and gC_part
    // (ndb, ..., N), gdt_part (ns, ..., 1).
    int nnb, ndb, ns;
    float *gx_part, *gB_part, *gC_part, *gdt_part;
    // In_proj rows (the in_proj layouts): x, Bt, Ct, dt point at the x, Re B, Re C
    // and dt blocks of token (0, 0)'s row and gx, gB, gC, gdt at the same blocks of
    // the gradient rows; rows are tok_stride elements apart (float32, or bfloat16
    // in kLayoutProjBf16, where the pointers hold 16-bit elements), an imaginary
    // block starts H*N elements after its real block, and x (so its gradient) is
    // real.
    int64_t tok_stride;
};

// The state pass's planes are read only as 4 consecutive rows x 16 consecutive
// columns (the contraction index runs down the rows). A wave's shared-memory
// read is served in two halves of 32 lanes over 32 4-byte banks, and a bank
// used twice costs a whole extra pass; a row stride of 16 mod 32 puts the two
// rows of each half 16 banks apart.
SSD_DEVICE int psa(int row, int col) { return row * kStrideA + col; }

inline int64_t bwd_block_rows(int64_t chunk) { return chunk < kBwdMaxRows ? chunk : kBwdMaxRows; }

struct BwdPlan {
    int R = 0, Q = 0, nc = 0, nnb = 1, ndb = 1, ns = 1;
    size_t states_bytes = 0, part_bytes = 0, gx_part_bytes = 0, bc_part_bytes = 0,
           gdt_part_bytes = 0, workspace_bytes = 0;
};

inline BwdPlan make_bwd_plan(int64_t B, int64_t T, int64_t H, int64_t N, int64_t D, int64_t chunk)
{
    BwdPlan p;
    p.Q = (int)bwd_block_rows(chunk);
    p.R = p.Q <= 16 ? 16 : 32;
    p.nc = (int)((T + p.Q - 1) / p.Q);
    p.nnb = (int)((N + 63) / 64);
    p.ndb = (int)((D + 63) / 64);
    p.ns = p.nnb * p.ndb;
    p.states_bytes = align_up((size_t)B * H * p.ns * p.nc * kStateFloats * 4, 256);
    p.part_bytes = align_up((size_t)B * H * p.ns * p.nc * 8, 256);
    if (p.ns > 1) {
        p.gx_part_bytes = align_up((size_t)p.nnb * B * T * H * D * 8, 256);
        p.bc_part_bytes = align_up((size_t)p.ndb * B * T * H * N * 8, 256);
        p.gdt_part_bytes = align_up((size_t)p.ns * B * T * H * 4, 256);
    }
    p.workspace_bytes = 2 * p.states_bytes + p.part_bytes + p.gx_part_bytes +
                        2 * p.bc_part_bytes + p.gdt_part_bytes;
    return p;
}

// A virtual sequence vs = seq * ns + slice: its (b, h), the slice's first state
// row n0 and column d0, and how many of its 64 rows and columns exist.
struct BwdSlice {
    int64_t seq;
    int st, n0, d0, nsl, dsl;
};
SSD_DEVICE BwdSlice bwd_slice(const BwdParams &p, int64_t vs)
{
    BwdSlice r;
    const uint32_t v = (uint32_t)vs, ns = (uint32_t)p.ns;  // vs < 2^31 (host check)
    r.seq = v / ns;
    r.st = (int)(v - (uint32_t)r.seq * ns);
    r.n0 = 64 * (r.st / p.ndb);
    r.d0 = 64 * (r.st % p.ndb);
    r.nsl = p.N - r.n0 < 64 ? p.N - r.n0 : 64;
    r.dsl = p.D - r.d0 < 64 ? p.D - r.d0 : 64;
    return r;
}

SSD_DEVICE v2f ld_c(const float *p, int64_t i) { return *(const v2f *)&p[2 * i]; }

// Complex product with its rounding fixed by explicit fused multiply-adds
// (the compiler may not contract it differently at different call sites): the
// adjoint pass and the fused chunk pass form the adjoint's update from it and
// so produce the same bits.
SSD_DEVICE v2f cmul_fixed(v2f a, v2f b)
{
    return v2f{fmaf(a.x, b.x, -(a.y * b.y)), fmaf(a.x, b.y, a.y * b.x)};
}
SSD_DEVICE v2f cmul_d(v2f a, v2f b) { return cmul(a, b); }

// Flat element index of (b, t, h, col) in a (B, T, H, width) tensor, or in
// the block of an in_proj row (the in_proj layouts).
template <int LAYOUT>
SSD_DEVICE int64_t bwd_elem(const BwdParams &p, int b, int t, int h, int width, int col)
{
    if constexpr (LAYOUT != kLayoutC64)
        return ((int64_t)b * p.T + t) * p.tok_stride + (int64_t)h * width + col;
    else
        return (((int64_t)b * p.T + t) * p.H + h) * width + col;
}

// Element e of an in_proj row array as loaded: a float32 value, or the 16 bits
// of a bfloat16 value held in a float register. The prefetch registers keep
// what was loaded; bwd_widen turns it into float32 where it is used, so that no
// conversion right behind a load makes the wave wait for that load.
template <int LAYOUT>
SSD_DEVICE float bwd_row_load(const float *base, int64_t e)
{
    if constexpr (LAYOUT == kLayoutProjBf16)
        return __builtin_bit_cast(float, (uint32_t)((const uint16_t *)base)[e]);
    else
        return base[e];
}
template <int LAYOUT>
SSD_DEVICE float bwd_widen(float v)
{
    if constexpr (LAYOUT == kLayoutProjBf16)
        return bf16_lo(__builtin_bit_cast(uint32_t, v));
    else
        return v;
}
template <int LAYOUT>
SSD_DEVICE v2f bwd_widen2(v2f v)
{
    return v2f{bwd_widen<LAYOUT>(v.x), bwd_widen<LAYOUT>(v.y)};
}

// float32 -> bfloat16, rounded to nearest with ties to even (NaN stays a quiet NaN).
SSD_DEVICE uint16_t f32_to_bf16(float v)
{
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x40u);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// Stores element e of an in_proj gradient row array (bfloat16 rounds).
template <int LAYOUT>
SSD_DEVICE void bwd_row_store(float *base, int64_t e, float v)
{
    if constexpr (LAYOUT == kLayoutProjBf16)
        ((uint16_t *)base)[e] = f32_to_bf16(v);
    else
        base[e] = v;
}

// Complex B_t or C_t element (base = p.Bt or p.Ct).
template <int LAYOUT>
SSD_DEVICE v2f bwd_load_bc(const BwdParams &p, const float *base, int b, int t, int h, int col)
{
    const int64_t e = bwd_elem<LAYOUT>(p, b, t, h, p.N, col);
    if constexpr (LAYOUT != kLayoutC64)
        return v2f{bwd_row_load<LAYOUT>(base, e), bwd_row_load<LAYOUT>(base, e + (int64_t)p.H * p.N)};
    else
        return ld_c(base, e);
}

// x element (real in the in_proj rows).
template <int LAYOUT>
SSD_DEVICE v2f bwd_load_x(const BwdParams &p, int b, int t, int h, int col)
{
    const int64_t e = bwd_elem<LAYOUT>(p, b, t, h, p.D, col);
    if constexpr (LAYOUT != kLayoutC64)
        return v2f{bwd_row_load<LAYOUT>(p.x, e), 0.f};
    else
        return ld_c(p.x, e);
}

// dt of chunk row tid (tid < R), or 0 past the chunk or past T (as loaded:
// bwd_widen gives the value). Every lane loads, through a buffer resource that
// ends after the chunk's last row, so lanes past it read zero and no branch
// makes the wave wait on the load.
template <int R, int LAYOUT>
SSD_DEVICE float bwd_load_dt(const BwdParams &p, int b, int h, int c)
{
    const int lane = thread_id() & 63;  // every wave holds the chunk's dt in lanes < R
    const int t0 = c * p.Q;
    int rows = p.T - t0 < p.Q ? p.T - t0 : p.Q;
    rows = rows < R ? rows : R;
    constexpr uint32_t es = LAYOUT == kLayoutProjBf16 ? 2u : 4u;  // bytes per element
    const uint32_t step = (uint32_t)(LAYOUT != kLayoutC64 ? p.tok_stride : p.H) * es;
    const buf_t r = make_buf((const char *)p.dt + bwd_elem<LAYOUT>(p, b, t0, h, 1, 0) * es,
                             (uint32_t)(rows - 1) * step + es);
    const uint32_t off = lane < rows ? (uint32_t)lane * step : kBwdOut;
    if constexpr (LAYOUT == kLayoutProjBf16)
        return __builtin_bit_cast(float, buf_load_u16(r, off));
    else
        return buf_load1(r, off);
}

// Double-precision lane moves (two 32-bit DPP / readlane moves).
template <int n>
SSD_DEVICE double row_shr_d(double v)
{
    const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
    const unsigned lo = (unsigned)row_shr_i<n>((int)(unsigned)u);
    const unsigned hi = (unsigned)row_shr_i<n>((int)(unsigned)(u >> 32));
    return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
}
SSD_DEVICE double lane_read_d(double v, int src)
{
    const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
    const unsigned lo = (unsigned)lane_read_i((int)(unsigned)u, src);
    const unsigned hi = (unsigned)lane_read_i((int)(unsigned)(u >> 32), src);
    return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
}

// Inclusive prefix sum over lanes 0..31 (a fixed tree: doubling inside each
// row of 16 lanes, then the first row's total added to the second row).
SSD_DEVICE double prefix32_d(double v)
{
    v += row_shr_d<1>(v);
    v += row_shr_d<2>(v);
    v += row_shr_d<4>(v);
    v += row_shr_d<8>(v);
    const double first = lane_read_d(v, 15);
    return (thread_id() & 63) >= 16 ? v + first : v;
}

// Called by all 64 lanes of one wave: lane l < R gets a_l = softplus(dt_l) A
// of chunk c (0 past the chunk or past T; dtv is lane l's dt) and its running
// sum lam (double); lam_end is the running sum at row R - 1, in every lane.
template <int R>
SSD_DEVICE void wave_decays(const BwdParams &p, int c, float dtv, float Ar, float Ai, double &lr,
                            double &li, double &er, double &ei)
{
    const int l = thread_id() & 63;
    const int t = c * p.Q + l;
    const bool valid = l < R && l < p.Q && t < p.T;
    const float sp = valid ? softplus_f(dtv) : 0.f;
    lr = prefix32_d((double)(sp * Ar));
    li = prefix32_d((double)(sp * Ai));
    er = lane_read_d(lr, R - 1);
    ei = lane_read_d(li, R - 1);
}

// exp of the difference of two running sums (taken in double, then rounded).
SSD_DEVICE v2f cexp_diff(const double *sLam, int l, int s)
{
    const double dr = (l >= 0 ? sLam[2 * l] : 0.0) - (s >= 0 ? sLam[2 * s] : 0.0);
    const double di = (l >= 0 ? sLam[2 * l + 1] : 0.0) - (s >= 0 ? sLam[2 * s + 1] : 0.0);
    return cexp_f(v2f{(float)dr, (float)di});
}

// ------------------------------------------------------- state and adjoint passes

// One workgroup per (b, h) walks the chunks (left to right for the state,
// right to left for the adjoint) and writes the value that enters (state) or
// leaves (adjoint) each chunk before folding the chunk in. The 64 x 64 value
// lives in MFMA accumulators: wave w holds tiles w and w + 8 of the 4 x 4 grid
// (rows n, columns d).
// Four waves per SIMD (two workgroups per CU, one staging while the other runs
// its MFMAs): at most 128 registers.
template <int R, bool REV, int LAYOUT>
SSD_KERNEL_WAVES(512, 4) void bwd_state_kernel(BwdParams p)
{
    // The update's right operand is complex only for the forward state from
    // complex64 tensors; it then takes three real products per complex one
    // (Gauss's form, as the scan): with a = f o B and x,
    //   k1 = (a_re + a_im) x_re,  k2 = a_im (x_re + x_im),  k3 = a_re (x_im - x_re),
    //   re += k1 - k2,  im += k1 + k3,
    // k1 summed over the chunk apart from the carried state and added to both at
    // the end. grad_y and in_proj's x are real: two products.
    constexpr bool CPLX = !REV && LAYOUT == kLayoutC64;
    constexpr int XP = CPLX ? R * kStrideA : 1;
    SSD_LDS float sAre[R * kStrideA];
    SSD_LDS float sAim[R * kStrideA];
    SSD_LDS float sAsum[XP];  // a_re + a_im
    SSD_LDS float sXre[R * kStrideA];
    SSD_LDS float sXn[XP];    // -(x_re + x_im)
    SSD_LDS float sXd[XP];    // x_im - x_re
    SSD_LDS float sF[2 * R];
    SSD_LDS float sDec[2];

    const int tid = thread_id();
    const int lane = tid & 63;
    const int w = wave_id();
    const int64_t vseq = block_id();  // (b, h) and state block
    const BwdSlice sl = bwd_slice(p, vseq);
    const int64_t seq = sl.seq;
    const int b = (int)(seq / p.H), h = (int)(seq % p.H);
    const float Ar = p.A[2 * h], Ai = p.A[2 * h + 1];
    const int N = sl.nsl, D = sl.dsl;  // rows and columns of this state block
    const int n0 = sl.n0, d0 = sl.d0;

    v4f sre[2], sim[2];
    for (int k = 0; k < 2; ++k) {
        const int idx = w + 8 * k, nt = idx >> 2, dtl = idx & 3;
        const int d = dtl * 16 + (lane & 15);
        for (int r = 0; r < 4; ++r) {
            const int n = nt * 16 + 4 * (lane >> 4) + r;
            v2f v = v2f{0.f, 0.f};
            const float *src = REV ? p.gfinal : p.init;
            if (src && n < N && d < D)
                v = ld_c(src, (seq * p.N + n0 + n) * p.D + d0 + d);
            sre[k][r] = v.x;
            sim[k][r] = REV ? -v.y : v.y;
        }
    }

    // The rows of the next chunk are loaded into registers while the current
    // chunk's MFMA update runs: PER elements of each operand per thread. For
    // complex64 tensors (VEC) through buffer resources: B_t or C_t as 16-byte
    // pairs (PB per thread), x or grad_y per element, with fixed lane offsets and
    // no conditions (rows past the chunk or T and columns past the block read zero).
    constexpr bool VEC = LAYOUT == kLayoutC64;
    constexpr int PER = R * 64 / 512;
    constexpr int PB = R / 16;
    v2f pa[PER], px[PER];
    v4f va[PB];
    float pdt = 0.f;
    const uint32_t rowN = (uint32_t)p.H * p.N * 8u, rowD = (uint32_t)p.H * p.D * 8u;
    const uint32_t rowG = (uint32_t)p.H * p.D * 4u;
    auto fetch = [&](int c) {
        pdt = bwd_load_dt<R, LAYOUT>(p, b, h, c);
        if constexpr (VEC) {
            const int64_t rows0 = ((int64_t)b * p.T + (int64_t)c * p.Q) * p.H + h;
            const int rv = p.T - c * p.Q < p.Q ? p.T - c * p.Q : p.Q;
            const buf_t ra = make_buf((REV ? p.Ct : p.Bt) + (rows0 * p.N + n0) * 2,
                                      (uint32_t)(rv - 1) * rowN + (uint32_t)N * 8u);
            for (int j = 0; j < PB; ++j) {
                const int e = tid + 512 * j, l = e >> 5, cp = e & 31;
                va[j] = buf_load4(ra, 2 * cp < N ? (uint32_t)l * rowN + 16u * cp : kBwdOut);
            }
            if (REV) {
                const buf_t rg = make_buf(p.gy + rows0 * p.D + d0,
                                          (uint32_t)(rv - 1) * rowG + (uint32_t)D * 4u);
                for (int j = 0; j < PER; ++j) {
                    const int i = tid + 512 * j, l = i >> 6, col = i & 63;
                    px[j] = v2f{buf_load1(rg, col < D ? (uint32_t)l * rowG + 4u * col : kBwdOut), 0.f};
                }
            } else {
                const buf_t rx = make_buf(p.x + (rows0 * p.D + d0) * 2,
                                          (uint32_t)(rv - 1) * rowD + (uint32_t)D * 8u);
                for (int j = 0; j < PER; ++j) {
                    const int i = tid + 512 * j, l = i >> 6, col = i & 63;
                    px[j] = buf_load2(rx, col < D ? (uint32_t)l * rowD + 8u * col : kBwdOut);
                }
            }
            return;
        }
        for (int j = 0; j < PER; ++j) {
            const int i = tid + 512 * j, l = i >> 6, col = i & 63;
            const int t = c * p.Q + l;
            // every lane loads (from a clamped element); the stage zeroes the lanes
            // outside the chunk, so no branch or select waits behind the loads
            const int tc = t < p.T ? t : p.T - 1;
            pa[j] = bwd_load_bc<LAYOUT>(p, REV ? p.Ct : p.Bt, b, tc, h, n0 + (col < N ? col : N - 1));
            if (REV)
                px[j] = v2f{p.gy[(((int64_t)b * p.T + tc) * p.H + h) * p.D + d0 +
                                 (col < D ? col : D - 1)],
                            0.f};
            else
                px[j] = bwd_load_x<LAYOUT>(p, b, tc, h, d0 + (col < D ? col : D - 1));
        }
    };
    fetch(REV ? p.nc - 1 : 0);

    for (int ci = 0; ci < p.nc; ++ci) {
        const int c = REV ? p.nc - 1 - ci : ci;
        float *slot = (REV ? p.adj_states : p.fwd_states) + (vseq * p.nc + c) * (int64_t)kStateFloats;
        const buf_t rslot = make_buf(slot, (uint32_t)kStateFloats * 4u);
        for (int k = 0; k < 2; ++k) {
            const int idx = w + 8 * k, nt = idx >> 2, dtl = idx & 3;
            const int d = dtl * 16 + (lane & 15);
            for (int r = 0; r < 4; ++r) {
                const int n = nt * 16 + 4 * (lane >> 4) + r;
                buf_store2(rslot, 8u * (uint32_t)(n * 64 + d), v2f{sre[k][r], sim[k][r]});
            }
        }
        if (w == 0) {
            // REV: e_in = exp(Lam[l]); forward: e_end = exp(Lam[R-1] - Lam[l])
            double lr, li, er, ei;
            wave_decays<R>(p, c, bwd_widen<LAYOUT>(pdt), Ar, Ai, lr, li, er, ei);
            if (lane < R)
                *(v2f *)&sF[2 * lane] = REV ? cexp_f(v2f{(float)lr, (float)li})
                                            : cexp_f(v2f{(float)(er - lr), (float)(ei - li)});
            if (lane == 0)
                *(v2f *)&sDec[0] = cexp_f(v2f{(float)er, (float)ei});
        }
        block_sync();
        if constexpr (VEC) {
            for (int j = 0; j < PB; ++j) {
                const int e = tid + 512 * j, l = e >> 5, c2 = 2 * (e & 31);
                const v2f f = *(const v2f *)&sF[2 * l];
                const v2f a0 = cmul_fixed(v2f{va[j].x, va[j].y}, f);
                const v2f a1 = cmul_fixed(v2f{va[j].z, va[j].w}, f);
                *(v2f *)&sAre[psa(l, c2)] = v2f{a0.x, a1.x};
                *(v2f *)&sAim[psa(l, c2)] = v2f{a0.y, a1.y};
                if constexpr (CPLX)
                    *(v2f *)&sAsum[psa(l, c2)] = v2f{a0.x + a0.y, a1.x + a1.y};
            }
            for (int j = 0; j < PER; ++j) {
                const int i = tid + 512 * j, l = i >> 6, col = i & 63;
                sXre[psa(l, col)] = px[j].x;
                if constexpr (CPLX) {
                    sXn[psa(l, col)] = -(px[j].x + px[j].y);
                    sXd[psa(l, col)] = px[j].y - px[j].x;
                }
            }
        }
        for (int j = 0; j < (VEC ? 0 : PER); ++j) {
            const int i = tid + 512 * j, l = i >> 6, col = i & 63;
            // REV: grad_y, always float32; otherwise x as loaded. Lanes outside the
            // chunk (or past N, D) are zeroed here.
            const int t = c * p.Q + l;
            const bool valid = l < p.Q && t < p.T;
            const v2f av = valid && col < N ? bwd_widen2<LAYOUT>(pa[j]) : v2f{0.f, 0.f};
            const v2f xv = !(valid && col < D) ? v2f{0.f, 0.f}
                                               : (REV ? px[j] : bwd_widen2<LAYOUT>(px[j]));
            const v2f a = cmul_fixed(av, *(const v2f *)&sF[2 * l]);
            sAre[psa(l, col)] = a.x;
            sAim[psa(l, col)] = a.y;
            sXre[psa(l, col)] = xv.x;  // real (grad_y, or in_proj's x)
        }
        block_sync();
        if (ci + 1 < p.nc)
            fetch(REV ? c - 1 : c + 1);
        const float dr = sDec[0], di = sDec[1];
        for (int k = 0; k < 2; ++k) {
            const int idx = w + 8 * k, nt = idx >> 2, dtl = idx & 3;
            v4f re, im;
            for (int r = 0; r < 4; ++r) {
                const v2f g = cmul_fixed(v2f{dr, di}, v2f{sre[k][r], sim[k][r]});
                re[r] = g.x;
                im[r] = g.y;
            }
            const int n = nt * 16 + (lane & 15);
            const int d = dtl * 16 + (lane & 15);
            v4f k1 = {0.f, 0.f, 0.f, 0.f};
            for (int l0 = 0; l0 < R; l0 += 4) {
                const int l = l0 + (lane >> 4);
                const float a_re = sAre[psa(l, n)], a_im = sAim[psa(l, n)];
                if constexpr (CPLX) {
                    const float a_s = sAsum[psa(l, n)];
                    const float x_re = sXre[psa(l, d)], x_n = sXn[psa(l, d)], x_d = sXd[psa(l, d)];
                    k1 = mfma_16x16x4(a_s, x_re, k1);
                    re = mfma_16x16x4(a_im, x_n, re);
                    im = mfma_16x16x4(a_re, x_d, im);
                } else {
                    const float g = sXre[psa(l, d)];
                    re = mfma_16x16x4(a_re, g, re);
                    im = mfma_16x16x4(a_im, g, im);
                }
            }
            if constexpr (CPLX) {
                re += k1;
                im += k1;
            }
            sre[k] = re;
            sim[k] = im;
        }
        block_sync();
    }

    if (REV && p.ginit) {
        for (int k = 0; k < 2; ++k) {
            const int idx = w + 8 * k, nt = idx >> 2, dtl = idx & 3;
            const int d = dtl * 16 + (lane & 15);
            for (int r = 0; r < 4; ++r) {
                const int n = nt * 16 + 4 * (lane >> 4) + r;
                if (n < N && d < D)
                    *(v2f *)&p.ginit[2 * ((seq * p.N + n0 + n) * p.D + d0 + d)] =
                        v2f{sre[k][r], -sim[k][r]};
            }
        }
    }
}

// ------------------------------------------------------------ the chunk pass

// Kinds of one MFMA step over a 4-wide K block: complex x complex (four MFMAs:
// rp += ar br, rn += ai bi, im += ar bi + ai br), real x complex (rp += a br,
// im += a bi), complex x real (rp += ar b, im += ai b) and real x real, or the
// real part alone of complex x real (rp += ar b). kCC3: complex x complex in three
// MFMAs, rp += ar br, rn += ai bi, im += (ar + ai)(br + bi), the product's imaginary
// part then being im - rp - rn.
enum { kCC = 0, kRC = 1, kCR = 2, kRR = 3, kCC3 = 4 };

// Steps k0 .. k1-1 of a tile product. ld(k) returns this lane's operands of
// step k as {ar, ai, br, bi}; the next step's operands are read from LDS before
// this step's MFMAs issue, so their latency hides behind the MFMAs.
template <int KIND, class Ld>
SSD_DEVICE void mma_steps(int k0, int k1, Ld ld, v4f &rp, v4f &rn, v4f &im)
{
    if (k0 >= k1)
        return;
    v4f cur = ld(k0);
    for (int k = k0; k < k1; ++k) {
        v4f nxt = cur;
        if (k + 1 < k1)
            nxt = ld(k + 1);
        sched_fence();
        if (KIND == kCC) {
            rp = mfma_16x16x4(cur.x, cur.z, rp);
            rn = mfma_16x16x4(cur.y, cur.w, rn);
            im = mfma_16x16x4(cur.x, cur.w, im);
            im = mfma_16x16x4(cur.y, cur.z, im);
        } else if (KIND == kCC3) {
            rp = mfma_16x16x4(cur.x, cur.z, rp);
            rn = mfma_16x16x4(cur.y, cur.w, rn);
            im = mfma_16x16x4(cur.x + cur.y, cur.z + cur.w, im);
        } else if (KIND == kRC) {
            rp = mfma_16x16x4(cur.x, cur.z, rp);
            im = mfma_16x16x4(cur.x, cur.w, im);
        } else if (KIND == kCR) {
            rp = mfma_16x16x4(cur.x, cur.z, rp);
            im = mfma_16x16x4(cur.y, cur.z, im);
        } else {
            rp = mfma_16x16x4(cur.x, cur.z, rp);
        }
        sched_fence();
        cur = nxt;
    }
}

// Sum over the 16 lanes of each row of a 16 x 16 accumulator tile: lane 15 of
// each group of 16 ends with the total of its 4 rows (inclusive prefix sums).
SSD_DEVICE v4f row_total(v4f v)
{
    for (int r = 0; r < 4; ++r) {
        float s = v[r];
        s += row_shr<1>(s);
        s += row_shr<2>(s);
        s += row_shr<4>(s);
        s += row_shr<8>(s);
        v[r] = s;
    }
    return v;
}

// Every chunk is independent given the stored entering states and leaving
// adjoints. A fixed number of workgroups (about one per compute unit) take the
// chunks in a strided loop, loading the next chunk's inputs into registers
// while the current one is evaluated.
//
// FUSED (at least as many sequences as workgroups, any input layout): no
// stored adjoints. Each workgroup takes whole (virtual) sequences and walks
// their chunks from the last to the first, keeping the adjoint G in the shared
// planes: it starts from conj(grad_final), and after a chunk's output tiles the
// waves fold the chunk in, G <- exp(Lam[R-1]) G + (e_in o C)^T gy -- the
// adjoint pass's update, in the same order and rounding, so the gradients are
// the same bits -- and after the first chunk they write the initial-state
// gradient.
template <int R, int LAYOUT, bool SLICED, bool FUSED>
SSD_KERNEL(512) void bwd_chunk_kernel(BwdParams p)
{
    constexpr int LD = kBwdLd;
    constexpr int SL = kStLd;
    constexpr int RL = R + 1;
    constexpr int NT = R / 16;                   // row tiles of the chunk
    constexpr int NPAIR = NT * (NT + 1) / 2;     // causal tile pairs
    SSD_LDS float sBre[R * LD];
    SSD_LDS float sBim[R * LD];
    SSD_LDS float sCre[R * LD];
    SSD_LDS float sCim[R * LD];
    SSD_LDS float sXre[R * LD];
    SSD_LDS float sXim[R * LD];
    SSD_LDS float sGy[R * LD];
    SSD_LDS float sHre[64 * SL];
    SSD_LDS float sHim[64 * SL];
    SSD_LDS float sGre[64 * SL];
    SSD_LDS float sGim[64 * SL];
    SSD_LDS float sMre[R * RL];
    SSD_LDS float sMim[R * RL];
    SSD_LDS float sVre[R * RL];
    SSD_LDS float sVim[R * RL];
    // running sums, dt and <H, G> partial sums of a chunk, in two slots: a chunk's
    // decay gradients are taken while the next chunk starts
    SSD_LDS double sLam[2][2 * R];
    SSD_LDS float sDt[2][R];
    SSD_LDS float sEin[2 * R];
    SSD_LDS float sEend[2 * R];
    // R = 32: exp(Lam[l] - Lam[15]) for l >= 16 and exp(Lam[15] - Lam[s]) for s < 16,
    // whose products are the decays of the pairs (l >= 16, s < 16)
    SSD_LDS float sFac[2 * R];
    SSD_LDS float sRow[3 * 4 * 2 * R];  // [O + Off, I, In][column tile][row] complex
    SSD_LDS float sTc[2][16];
    SSD_LDS float sEv[2 * R];  // per row: (O - I + Off) and In, all column tiles
    SSD_LDS float sEe[2 * R];
    SSD_LDS float sVd[2 * R];  // the diagonal V[l][l], kept out of the V tiles

    const int tid = thread_id();
    const int lane = tid & 63;
    const int w = wave_id();
    const int64_t total = (int64_t)p.B * p.H * p.ns * p.nc;
    const int64_t nvseq = (int64_t)p.B * p.H * p.ns;

    // The next chunk's inputs are loaded into registers while the current one
    // is evaluated (PER row elements and PS state elements per thread). For
    // complex64 tensors (VEC) B_t, C_t and the stored states move as 16-byte
    // groups of two complex values (PB and PSV groups per thread), x and grad_y
    // per element, all through buffer resources: each chunk moves the resource
    // bases, the lane offsets stay, and every load is unconditional (rows past
    // the chunk or T and columns past the slice lie outside the resource and
    // read zero).
    constexpr bool VEC = LAYOUT == kLayoutC64;
    constexpr int PER = R * 64 / 512;
    constexpr int PS = 64 * 64 / 512;
    constexpr int PB = R / 16;
    constexpr int PSV = 4;
    v2f pb[PER], pc[PER], px[PER], ph[PS], pg[PS];
    v4f vb[PB], vc[PB], vh[PSV], vg[PSV];
    float pgy[PER];
    float pdt = 0.f;
    const uint32_t rowN = (uint32_t)p.H * p.N * 8u;  // bytes between token rows of B_t, C_t
    const uint32_t rowD = (uint32_t)p.H * p.D * 8u;  // ... of x
    const uint32_t rowG = (uint32_t)p.H * p.D * 4u;  // ... of grad_y
    // fetch(part, k): part 0 = dt, B_t and C_t rows; 1 = x and grad_y rows;
    // 2 = the entering state; 3 = the leaving adjoint. The parts of the next
    // chunk are issued at different points of the current one, so that no
    // wave stalls behind a long burst of loads.
    // Where chunk k lies: its index in the sequence, the (virtual) sequence's
    // state block, batch row and head, from 32-bit divisions (the host keeps the
    // (virtual sequence, chunk) count below 2^31), worked out once per chunk.
    struct Pos {
        int64_t k, vs;  // chunk, virtual sequence
        int c, b, h;
        BwdSlice ks;
    };
    auto pos_of = [&](int64_t k) {
        Pos r;
        r.k = k;
        const uint32_t ku = (uint32_t)k, nc = (uint32_t)p.nc;
        const uint32_t vs = (uint32_t)uniform_i((int)(ku / nc));
        r.vs = vs;
        r.c = (int)(ku - vs * nc);
        r.ks = SLICED ? bwd_slice(p, vs) : BwdSlice{(int64_t)vs, 0, 0, 0, p.N, p.D};
        const uint32_t sq = (uint32_t)r.ks.seq, nh = (uint32_t)p.H;
        r.b = uniform_i((int)(sq / nh));
        r.h = (int)(sq - (uint32_t)r.b * nh);
        return r;
    };
    // fetch(part, pos): part 0 = dt, B_t and C_t rows; 1 = x and grad_y rows;
    // 2 = the entering state; 3 = the leaving adjoint. The parts of the next
    // chunk are issued at different points of the current one, so that no
    // wave stalls behind a long burst of loads.
    auto fetch = [&](auto part_c, const Pos &pos) {
        constexpr int part = decltype(part_c)::value;
        const int64_t k = pos.k;
        const int cc = pos.c;
        const BwdSlice ks = pos.ks;
        const int bb = pos.b, hh = pos.h;
        if constexpr (part == 0)
            pdt = bwd_load_dt<R, LAYOUT>(p, bb, hh, cc);
        if constexpr (VEC) {
            const int64_t rows0 = ((int64_t)bb * p.T + (int64_t)cc * p.Q) * p.H + hh;
            const int rv = p.T - cc * p.Q < p.Q ? p.T - cc * p.Q : p.Q;  // rows that exist
            if constexpr (part == 0) {
                const uint32_t nb = (uint32_t)(rv - 1) * rowN + (uint32_t)ks.nsl * 8u;
                const buf_t rb = make_buf(p.Bt + (rows0 * p.N + ks.n0) * 2, nb);
                const buf_t rc = make_buf(p.Ct + (rows0 * p.N + ks.n0) * 2, nb);
                for (int j = 0; j < PB; ++j) {
                    const int e = tid + 512 * j, l = e >> 5, cp = e & 31;
                    const uint32_t off = 2 * cp < ks.nsl ? (uint32_t)l * rowN + 16u * cp : kBwdOut;
                    vb[j] = buf_load4(rb, off);
                    vc[j] = buf_load4(rc, off);
                }
            } else if constexpr (part == 1) {
                const buf_t rx = make_buf(p.x + (rows0 * p.D + ks.d0) * 2,
                                          (uint32_t)(rv - 1) * rowD + (uint32_t)ks.dsl * 8u);
                const buf_t rg = make_buf(p.gy + rows0 * p.D + ks.d0,
                                          (uint32_t)(rv - 1) * rowG + (uint32_t)ks.dsl * 4u);
                for (int j = 0; j < PER; ++j) {
                    const int i = tid + 512 * j, l = i >> 6, col = i & 63;
                    const bool in = col < ks.dsl;
                    px[j] = buf_load2(rx, in ? (uint32_t)l * rowD + 8u * col : kBwdOut);
                    pgy[j] = buf_load1(rg, in ? (uint32_t)l * rowG + 4u * col : kBwdOut);
                }
            } else if constexpr (FUSED && part == 3) {
                // the adjoint is walked in shared memory (grad_final is read where a
                // sequence's first chunk is staged)
            } else {
                const float *src = (part == 2 ? p.fwd_states : p.adj_states) + k * (int64_t)kStateFloats;
                const buf_t rs = make_buf(src, (uint32_t)kStateFloats * 4u);
                for (int j = 0; j < PSV; ++j) {
                    if constexpr (part == 2)
                        vh[j] = buf_load4(rs, 16u * (tid + 512 * j));
                    else
                        vg[j] = buf_load4(rs, 16u * (tid + 512 * j));
                }
            }
        } else if constexpr (part <= 1) {
            for (int j = 0; j < PER; ++j) {
                const int i = tid + 512 * j, l = i >> 6, col = i & 63;
                const int t = cc * p.Q + l;
                const bool valid = l < p.Q && t < p.T;
                const int64_t row = ((int64_t)bb * p.T + t) * p.H + hh;
                const bool vn = valid && col < ks.nsl, vd = valid && col < ks.dsl;
                if constexpr (part == 0) {
                    pb[j] = vn ? bwd_load_bc<LAYOUT>(p, p.Bt, bb, t, hh, ks.n0 + col) : v2f{0.f, 0.f};
                    pc[j] = vn ? bwd_load_bc<LAYOUT>(p, p.Ct, bb, t, hh, ks.n0 + col) : v2f{0.f, 0.f};
                } else {
                    px[j] = vd ? bwd_load_x<LAYOUT>(p, bb, t, hh, ks.d0 + col) : v2f{0.f, 0.f};
                    pgy[j] = vd ? p.gy[row * p.D + ks.d0 + col] : 0.f;
                }
            }
        } else if constexpr (!(FUSED && part == 3)) {
            const float *src = (part == 2 ? p.fwd_states : p.adj_states) + k * (int64_t)kStateFloats;
            for (int j = 0; j < PS; ++j) {
                if constexpr (part == 2)
                    ph[j] = ld_c(src, tid + 512 * j);
                else
                    pg[j] = ld_c(src, tid + 512 * j);
            }
        }
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using P2 = std::integral_constant<int, 2>;
    using P3 = std::integral_constant<int, 3>;
    // new_seq (FUSED): the staged chunk k is its sequence's last, so G starts from
    // conj(grad_final) (read here, once per sequence); otherwise the G planes
    // already hold the walked adjoint.
    auto stage = [&](bool new_seq, const Pos &pos) {
        if constexpr (FUSED) {
            if (new_seq) {
                const BwdSlice ks = pos.ks;
                const buf_t rf = make_buf(
                    p.gfinal ? p.gfinal + ((ks.seq * p.N + ks.n0) * p.D + ks.d0) * 2 : nullptr,
                    p.gfinal ? (uint32_t)((ks.nsl - 1) * p.D + ks.dsl) * 8u : 0u);
                for (int j = 0; j < 8; ++j) {
                    const int i = tid + 512 * j, n = i >> 6, d = i & 63;
                    const v2f g = buf_load2(rf, d < ks.dsl ? (uint32_t)(n * p.D + d) * 8u : kBwdOut);
                    sGre[n * SL + d] = g.x;
                    sGim[n * SL + d] = -g.y;
                }
            }
        }
        if constexpr (VEC) {
            for (int j = 0; j < PB; ++j) {
                const int e = tid + 512 * j, l = e >> 5, c2 = 2 * (e & 31);
                sBre[l * LD + c2] = vb[j].x;
                sBim[l * LD + c2] = vb[j].y;
                sBre[l * LD + c2 + 1] = vb[j].z;
                sBim[l * LD + c2 + 1] = vb[j].w;
                sCre[l * LD + c2] = vc[j].x;
                sCim[l * LD + c2] = vc[j].y;
                sCre[l * LD + c2 + 1] = vc[j].z;
                sCim[l * LD + c2 + 1] = vc[j].w;
            }
            for (int j = 0; j < PER; ++j) {
                const int i = tid + 512 * j, l = i >> 6, col = i & 63;
                sXre[l * LD + col] = px[j].x;
                sXim[l * LD + col] = px[j].y;
                sGy[l * LD + col] = pgy[j];
            }
            for (int j = 0; j < PSV; ++j) {
                const int e = tid + 512 * j, n = e >> 5, d2 = 2 * (e & 31);
                sHre[n * SL + d2] = vh[j].x;
                sHim[n * SL + d2] = vh[j].y;
                sHre[n * SL + d2 + 1] = vh[j].z;
                sHim[n * SL + d2 + 1] = vh[j].w;
                if constexpr (!FUSED) {
                    sGre[n * SL + d2] = vg[j].x;
                    sGim[n * SL + d2] = vg[j].y;
                    sGre[n * SL + d2 + 1] = vg[j].z;
                    sGim[n * SL + d2 + 1] = vg[j].w;
                }
            }
            return;
        }
        for (int j = 0; j < PER; ++j) {
            const int i = tid + 512 * j, l = i >> 6, col = i & 63;
            const v2f bv = bwd_widen2<LAYOUT>(pb[j]), cv = bwd_widen2<LAYOUT>(pc[j]);
            const v2f xv = bwd_widen2<LAYOUT>(px[j]);
            sBre[l * LD + col] = bv.x;
            sBim[l * LD + col] = bv.y;
            sCre[l * LD + col] = cv.x;
            sCim[l * LD + col] = cv.y;
            sXre[l * LD + col] = xv.x;
            sXim[l * LD + col] = xv.y;
            sGy[l * LD + col] = pgy[j];
        }
        for (int j = 0; j < PS; ++j) {
            const int i = tid + 512 * j, n = i >> 6, d = i & 63;
            sHre[n * SL + d] = ph[j].x;
            sHim[n * SL + d] = ph[j].y;
            if constexpr (!FUSED) {
                sGre[n * SL + d] = pg[j].x;
                sGim[n * SL + d] = pg[j].y;
            }
        }
    };

    // The chunk after chunk k in this workgroup's order, or -1.
    auto next_of = [&](const Pos &pos) -> int64_t {
        if constexpr (FUSED) {
            if (pos.c > 0)
                return pos.k - 1;
            const int64_t vs = pos.vs + grid_blocks();
            return vs < nvseq ? vs * p.nc + p.nc - 1 : -1;
        } else {
            const int64_t n = pos.k + grid_blocks();
            return n < total ? n : -1;
        }
    };
    // Decay gradients of chunk k (one wave): its row sums sEv, sEe (kept until the
    // next chunk's output tiles), and its running sums, dt and <H, G> partial sums
    // in slot q.
    auto decay_grads = [&](const Pos &pos, int q) {
        const int64_t k = pos.k;
        const BwdSlice ks = pos.ks;
        const int kc = pos.c;
        const int kb = pos.b, kh = pos.h;
        const v2f kA = ld_c_uniform(p.A, kh);
        const float kAr = kA.x, kAi = kA.y;
            // dF/da_t = sum_{j>=t} v_j + sum_{j<t} In_j + exp(Lam[R-1]) <H, G>: the
            // suffix and prefix sums over the chunk rows as lane scans (fixed trees)
            const int t0 = lane;
            const bool row = t0 < R;
            float vr = row ? sEv[2 * t0] : 0.f, vi = row ? sEv[2 * t0 + 1] : 0.f;
            float er = row ? sEe[2 * t0] : 0.f, ei = row ? sEe[2 * t0 + 1] : 0.f;
            vr += row_shl<1>(vr);
            vi += row_shl<1>(vi);
            vr += row_shl<2>(vr);
            vi += row_shl<2>(vi);
            vr += row_shl<4>(vr);
            vi += row_shl<4>(vi);
            vr += row_shl<8>(vr);
            vi += row_shl<8>(vi);
            const float nr = lane_read(vr, 16), ni = lane_read(vi, 16);
            if (t0 < 16) {
                vr += nr;
                vi += ni;
            }
            er += row_shr<1>(er);
            ei += row_shr<1>(ei);
            er += row_shr<2>(er);
            ei += row_shr<2>(ei);
            er += row_shr<4>(er);
            ei += row_shr<4>(ei);
            er += row_shr<8>(er);
            ei += row_shr<8>(ei);
            float xr = row_shr<1>(er), xi = row_shr<1>(ei);  // exclusive
            const float pr = lane_read(er, 15), pi = lane_read(ei, 15);
            if (t0 >= 16) {
                xr += pr;
                xi += pi;
            }
            float tr = 0.f, ti = 0.f;
            for (int i = 0; i < 8; ++i) {
                tr += sTc[q][2 * i];
                ti += sTc[q][2 * i + 1];
            }
            const v2f Tc = cmul(cexp_diff(sLam[q], R - 1, -1), v2f{tr, ti});
            const float fr = (vr + xr) + Tc.x, fi = (vi + xi) + Tc.y;
            float gAr = 0.f, gAi = 0.f;
            const int t = kc * p.Q + t0;
            if (row && t0 < p.Q && t < p.T) {
                // ga = conj(dF/da)
                const float gar = fr, gai = -fi;
                const float dtv = sDt[q][t0];
                const float sig = 1.f / (1.f + expf(-dtv));
                if constexpr (SLICED)
                    p.gdt_part[((int64_t)ks.st * p.B * p.T + (int64_t)kb * p.T + t) * p.H + kh] =
                        (kAr * gar + kAi * gai) * sig;
                else
                    bwd_row_store<LAYOUT>(p.gdt, bwd_elem<LAYOUT>(p, kb, t, kh, 1, 0),
                                          (kAr * gar + kAi * gai) * sig);
                const float sp = softplus_f(dtv);
                gAr = sp * gar;
                gAi = sp * gai;
            }
            // this chunk's share of gA: a fixed-order sum over the wave
            gAr += row_shr<1>(gAr);
            gAr += row_shr<2>(gAr);
            gAr += row_shr<4>(gAr);
            gAr += row_shr<8>(gAr);
            gAi += row_shr<1>(gAi);
            gAi += row_shr<2>(gAi);
            gAi += row_shr<4>(gAi);
            gAi += row_shr<8>(gAi);
            const float r0 = lane_read(gAr, 15), r1 = lane_read(gAr, 31);
            const float i0 = lane_read(gAi, 15), i1 = lane_read(gAi, 31);
            if (lane == 0)
                *(v2f *)&p.gA_part[2 * k] = v2f{r0 + r1, i0 + i1};
    };
    if (block_id() >= (FUSED ? nvseq : total))
        return;
    Pos cur = pos_of(FUSED ? block_id() * p.nc + p.nc - 1 : block_id());
    fetch(P0{}, cur);
    fetch(P1{}, cur);
    fetch(P2{}, cur);
    fetch(P3{}, cur);
    stage(true, cur);
    block_sync();
    int par = 0;         // slot of this chunk's running sums, dt and <H, G> sums
    Pos prev;            // the chunk whose decay gradients are still to be taken
    bool has_prev = false;
    for (;;) {
        const BwdSlice cs = cur.ks;
        const int64_t seq = cs.seq;
        const int c = cur.c;
        const int b = cur.b, h = cur.h;
        const v2f Ah = ld_c_uniform(p.A, h);
        const float Ar = Ah.x, Ai = Ah.y;
        if (w == kDecayWave) {
            // running sums and row factors of this chunk; read after the next barrier
            double lr, li, er, ei;
            const float dtv = bwd_widen<LAYOUT>(pdt);
            wave_decays<R>(p, c, dtv, Ar, Ai, lr, li, er, ei);
            const double mr = lane_read_d(lr, 15), mi = lane_read_d(li, 15);
            if (R == 32 && LAYOUT == kLayoutC64 && lane < R)
                *(v2f *)&sFac[2 * lane] = lane < 16 ? cexp_f(v2f{(float)(mr - lr), (float)(mi - li)})
                                                    : cexp_f(v2f{(float)(lr - mr), (float)(li - mi)});
            if (lane < R) {
                const int t = c * p.Q + lane;
                sLam[par][2 * lane] = lr;
                sLam[par][2 * lane + 1] = li;
                sDt[par][lane] = (lane < p.Q && t < p.T) ? dtv : 0.f;
                *(v2f *)&sEin[2 * lane] = cexp_f(v2f{(float)lr, (float)li});
                *(v2f *)&sEend[2 * lane] = cexp_f(v2f{(float)(er - lr), (float)(ei - li)});
            }
        }
        if (w == kGradWave && has_prev)
            decay_grads(prev, par ^ 1);
        const int64_t next = next_of(cur);
        const bool has_next = next >= 0;
        const Pos npos = pos_of(has_next ? next : cur.k);
        if (has_next)
            fetch(P0{}, npos);

        // Raw Gram (C B^T) tiles on waves 0.., raw gy x^T tiles on waves 4..
        if (w < NPAIR || (w >= 4 && w < 4 + NPAIR)) {
            const bool gram = w < 4;
            const int k = gram ? w : w - 4;
            const int lt = k < NT ? k : NT - 1, st = k < NT ? k : 0;  // (0,0), (1,1), (1,0)
            const int lrow = lt * 16 + (lane & 15), scol = st * 16 + (lane & 15);
            v4f rp = {0.f, 0.f, 0.f, 0.f}, rn = rp, im = rp;
            const int g4 = lane >> 4;
            if (gram) {
                // three MFMAs per step (Gauss's form): the Gram waves' SIMDs carry the
                // section's MFMAs, and this section holds few registers
                mma_steps<kCC3>(0, 16, [&](int k) {
                    const int kk = 4 * k + g4;
                    return v4f{sCre[lrow * LD + kk], sCim[lrow * LD + kk], sBre[scol * LD + kk],
                               sBim[scol * LD + kk]};
                }, rp, rn, im);
            } else if constexpr (LAYOUT == kLayoutC64) {
                mma_steps<kRC>(0, 16, [&](int k) {
                    const int kk = 4 * k + g4;
                    return v4f{sGy[lrow * LD + kk], 0.f, sXre[scol * LD + kk], sXim[scol * LD + kk]};
                }, rp, rn, im);
            } else {
                // in_proj's x is real: gy x^T is real
                mma_steps<kRR>(0, 16, [&](int k) {
                    const int kk = 4 * k + g4;
                    return v4f{sGy[lrow * LD + kk], 0.f, sXre[scol * LD + kk], 0.f};
                }, rp, rn, im);
            }
            float *dre = gram ? sMre : sVre;
            float *dim = gram ? sMim : sVim;
            for (int r = 0; r < 4; ++r) {
                const int l = lt * 16 + 4 * (lane >> 4) + r, s = st * 16 + (lane & 15);
                dre[l * RL + s] = rp[r] - rn[r];
                dim[l * RL + s] = gram ? im[r] - rp[r] - rn[r] : im[r];
            }
        }
        // <H, G> partial sums
        {
            float tr = 0.f, ti = 0.f;
            for (int i = tid; i < 64 * 64; i += 512) {
                const int n = i >> 6, d = i & 63;
                const float hr = sHre[n * SL + d], hi = sHim[n * SL + d];
                const float gr = sGre[n * SL + d], gi = sGim[n * SL + d];
                tr += hr * gr - hi * gi;
                ti += hr * gi + hi * gr;
            }
            tr += row_shr<1>(tr);
            tr += row_shr<2>(tr);
            tr += row_shr<4>(tr);
            tr += row_shr<8>(tr);
            ti += row_shr<1>(ti);
            ti += row_shr<2>(ti);
            ti += row_shr<4>(ti);
            ti += row_shr<8>(ti);
            const float t0r = lane_read(tr, 15), t1r = lane_read(tr, 31);
            const float t2r = lane_read(tr, 47), t3r = lane_read(tr, 63);
            const float t0i = lane_read(ti, 15), t1i = lane_read(ti, 31);
            const float t2i = lane_read(ti, 47), t3i = lane_read(ti, 63);
            if (lane == 0) {
                sTc[par][2 * w] = (t0r + t1r) + (t2r + t3r);
                sTc[par][2 * w + 1] = (t0i + t1i) + (t2i + t3i);
            }
        }
        block_sync();

        if (has_next) {
            fetch(P1{}, npos);
            fetch(P2{}, npos);
        }
        // M = Gram o L and V = (gy x^T) o L, zero above the diagonal. V's
        // diagonal goes to sVd and the V tiles hold only the pairs l > s: the
        // decay gradients sum row dots of the products with V, and a token's
        // pair with itself, which no decay multiplies, must not enter them (it
        // would cancel between two differently rounded sums). The output tiles
        // add the diagonal term back from sVd.
        // R = 32 (complex64 tensors), two passes of the 512 threads: first the two
        // diagonal 16 x 16 tiles (an exponential of a difference of running sums per
        // pair), then the tile below them (a product of the two factors in sFac) on
        // waves 0-3 and the zero tile above on waves 4-7. Otherwise every pair takes
        // its exponential (the in_proj variants hold more prefetch registers, and the
        // split pass would push them into spills).
        auto pair = [&](int l, int s, int how) {  // how: 0 exponential, 1 factors, 2 zero
            float mr = 0.f, mi = 0.f, vr = 0.f, vi = 0.f;
            if (how == 1 || (how == 0 && l >= s)) {
                const v2f L = how == 0 ? cexp_diff(sLam[par], l, s)
                                       : cmul(*(const v2f *)&sFac[2 * l], *(const v2f *)&sFac[2 * s]);
                const v2f m = cmul(v2f{sMre[l * RL + s], sMim[l * RL + s]}, L);
                const v2f v = cmul(v2f{sVre[l * RL + s], sVim[l * RL + s]}, L);
                mr = m.x;
                mi = m.y;
                vr = v.x;
                vi = v.y;
            }
            if (l == s) {
                *(v2f *)&sVd[2 * l] = v2f{vr, vi};
                vr = 0.f;
                vi = 0.f;
            }
            sMre[l * RL + s] = mr;
            sMim[l * RL + s] = mi;
            sVre[l * RL + s] = vr;
            sVim[l * RL + s] = vi;
        };
        if constexpr (R == 32 && LAYOUT == kLayoutC64) {
            const int e = tid & 255, hi = tid >> 8;  // hi: waves 4-7
            pair(16 * hi + (e >> 4), 16 * hi + (e & 15), 0);
            if (hi == 0)
                pair(16 + (e >> 4), e & 15, 1);
            else
                pair(e >> 4, 16 + (e & 15), 2);
        } else {
            for (int i = tid; i < R * R; i += 512)
                pair(i / R, i % R, 0);
        }
        block_sync();

        // Output tiles: gx (rows s, columns d), gB (rows s, columns n), gC (rows l,
        // columns n); NT x 4 tiles of each, dealt round-robin over the eight
        // waves. Each tile also leaves one row dot product for the decay
        // gradients (sRow slot q, column tile ct), with V's diagonal left out:
        //   gx: In_s = x_s . (e_end B G)_s                           (q = 2)
        //   gB: I_s  = B_s . (V^T C)_s  over l > s                    (q = 1)
        //   gC: (O + Off)_l = C_l . ((V B)_l over s < l + e_in (gy H^T)_l)  (q = 0)
        if (has_next)
            fetch(P3{}, npos);  // FUSED: grad_final when next starts a sequence, else nothing
        // Complex64 tensors: one body per kind (KC a compile-time kind), so each
        // epilogue carries only its own terms (-2.5 % per call). The in_proj layouts
        // keep one body for all kinds below: measured, the per-kind form pushes them
        // into register spills and costs them 10 %.
        auto c64_tile = [&](auto kc, int tile) {
            constexpr int kind = decltype(kc)::value;
            const int rt = (tile % (NT * 4)) >> 2, ct = tile & 3;
            const int arow = rt * 16 + (lane & 15);      // row this lane feeds as A
            const int bcol = ct * 16 + (lane & 15);      // column this lane feeds as B
            const int g4 = lane >> 4;
            v4f p2r = {0.f, 0.f, 0.f, 0.f}, p2n = p2r, p2i = p2r;  // edge term (re+, re-, im)
            v4f p1r = p2r, p1n = p2r, p1i = p2r;                   // in-chunk term
            if constexpr (kind == 0) {
                // conj(gx) = M^T gy + e_end (B G)
                mma_steps<kCC>(0, 16, [&](int k) {
                    const int n = 4 * k + g4;
                    return v4f{sBre[arow * LD + n], sBim[arow * LD + n], sGre[n * SL + bcol],
                               sGim[n * SL + bcol]};
                }, p2r, p2n, p2i);
                mma_steps<kCR>(rt * 4, R / 4, [&](int k) {
                    const int l = 4 * k + g4;
                    return v4f{sMre[l * RL + arow], sMim[l * RL + arow], sGy[l * LD + bcol], 0.f};
                }, p1r, p1n, p1i);
            } else if constexpr (kind == 1) {
                // conj(gB) = V^T C + e_end (x G^T)
                mma_steps<kCC>(0, 16, [&](int k) {
                    const int d = 4 * k + g4;
                    return v4f{sXre[arow * LD + d], sXim[arow * LD + d], sGre[bcol * SL + d],
                               sGim[bcol * SL + d]};
                }, p2r, p2n, p2i);
                mma_steps<kCC3>(rt * 4, R / 4, [&](int k) {
                    const int l = 4 * k + g4;
                    return v4f{sVre[l * RL + arow], sVim[l * RL + arow], sCre[l * LD + bcol],
                               sCim[l * LD + bcol]};
                }, p1r, p1n, p1i);
            } else {
                // conj(gC) = V B + e_in (gy H^T)
                mma_steps<kRC>(0, 16, [&](int k) {
                    const int d = 4 * k + g4;
                    return v4f{sGy[arow * LD + d], 0.f, sHre[bcol * SL + d], sHim[bcol * SL + d]};
                }, p2r, p2n, p2i);
                mma_steps<kCC3>(0, rt * 4 + 4, [&](int k) {
                    const int sx = 4 * k + g4;
                    return v4f{sVre[arow * RL + sx], sVim[arow * RL + sx], sBre[sx * LD + bcol],
                               sBim[sx * LD + bcol]};
                }, p1r, p1n, p1i);
            }
            if constexpr (kind != 0) {  // the in-chunk products' imaginary parts (kCC3)
                for (int r = 0; r < 4; ++r)
                    p1i[r] = p1i[r] - p1r[r] - p1n[r];
            }
            const int col = ct * 16 + (lane & 15);
            const float *fac = kind == 2 ? sEin : sEend;
            const float *qre = kind == 0 ? sXre : (kind == 1 ? sBre : sCre);
            const float *qim = kind == 0 ? sXim : (kind == 1 ? sBim : sCim);
            // the diagonal pair's term of gB (V[s][s] C_s) and gC (V[l][l] B_l)
            const float *ore = kind == 1 ? sCre : sBre;
            const float *oim = kind == 1 ? sCim : sBim;
            v4f outr, outi, dr, di;
            for (int r = 0; r < 4; ++r) {
                const int row = rt * 16 + 4 * (lane >> 4) + r;
                const v2f f = *(const v2f *)&fac[2 * row];
                const v2f e2 = cmul(f, v2f{p2r[r] - p2n[r], p2i[r]});
                const v2f e1 = v2f{p1r[r] - p1n[r], p1i[r]};
                const v2f vd = kind == 0 ? v2f{0.f, 0.f} : *(const v2f *)&sVd[2 * row];
                const v2f e0 = cmul(vd, v2f{ore[row * LD + col], oim[row * LD + col]});
                const v2f m = kind == 0 ? e2 : (kind == 1 ? e1 : v2f{e1.x + e2.x, e1.y + e2.y});
                outr[r] = (e1.x + e2.x) + e0.x;
                outi[r] = (e1.y + e2.y) + e0.y;
                const v2f q = v2f{qre[row * LD + col], qim[row * LD + col]};
                const v2f d = cmul(q, m);
                dr[r] = d.x;
                di[r] = d.y;
            }
            dr = row_total(dr);
            di = row_total(di);
            if ((lane & 15) == 15) {
                const int q = 2 - kind;
                for (int r = 0; r < 4; ++r) {
                    const int row = rt * 16 + 4 * (lane >> 4) + r;
                    sRow[((q * 4 + ct) * R + row) * 2] = dr[r];
                    sRow[((q * 4 + ct) * R + row) * 2 + 1] = di[r];
                }
            }
            const int width = kind == 0 ? p.D : p.N;
            const int cols = kind == 0 ? cs.dsl : cs.nsl;
            const int gcol = (kind == 0 ? cs.d0 : cs.n0) + col;
            if constexpr (!SLICED) {
                // straight-line stores: rows past the chunk or T and columns past
                // the width lie outside the resource and are dropped
                float *dst = kind == 0 ? p.gx : (kind == 1 ? p.gB : p.gC);
                const int64_t rows0 = ((int64_t)b * p.T + (int64_t)c * p.Q) * p.H + h;
                const int rv = p.T - c * p.Q < p.Q ? p.T - c * p.Q : p.Q;
                const uint32_t rowW = (uint32_t)p.H * width * 8u;
                const buf_t ro = make_buf(dst + rows0 * width * 2,
                                          (uint32_t)(rv - 1) * rowW + (uint32_t)cols * 8u);
                for (int r = 0; r < 4; ++r) {
                    const int row = rt * 16 + 4 * (lane >> 4) + r;
                    buf_store2(ro, col < cols ? (uint32_t)row * rowW + 8u * col : kBwdOut,
                               v2f{outr[r], -outi[r]});
                }
                return;
            }
            for (int r = 0; r < 4; ++r) {
                const int row = rt * 16 + 4 * (lane >> 4) + r;
                const int t = c * p.Q + row;
                if (row < p.Q && t < p.T && col < cols) {
                    if constexpr (SLICED) {
                        // partial over the other dimension's slices: gx over S, gB and
                        // gC over T, complex in the (B, T, H, width) layout
                        const int sl = kind == 0 ? cs.st / p.ndb : cs.st % p.ndb;
                        float *part = kind == 0 ? p.gx_part : (kind == 1 ? p.gB_part : p.gC_part);
                        const int64_t g = ((int64_t)b * p.T + t) * p.H + h;
                        const int64_t e = ((int64_t)sl * p.B * p.T * p.H + g) * width + gcol;
                        *(v2f *)&part[2 * e] = v2f{outr[r], -outi[r]};
                        continue;
                    }
                    float *dst = kind == 0 ? p.gx : (kind == 1 ? p.gB : p.gC);
                    const int64_t g = ((int64_t)b * p.T + t) * p.H + h;
                    *(v2f *)&dst[2 * (g * width + gcol)] = v2f{outr[r], -outi[r]};
                }
            }
        };
        for (int tile = w; tile < 3 * NT * 4; tile += 8) {
            const int kind = tile / (NT * 4);
            if constexpr (LAYOUT == kLayoutC64) {
                if (kind == 0)
                    c64_tile(std::integral_constant<int, 0>{}, tile);
                else if (kind == 1)
                    c64_tile(std::integral_constant<int, 1>{}, tile);
                else
                    c64_tile(std::integral_constant<int, 2>{}, tile);
            } else {
                const int rt = (tile % (NT * 4)) >> 2, ct = tile & 3;
                const int arow = rt * 16 + (lane & 15);      // row this lane feeds as A
                const int bcol = ct * 16 + (lane & 15);      // column this lane feeds as B
                const int g4 = lane >> 4;
                v4f p2r = {0.f, 0.f, 0.f, 0.f}, p2n = p2r, p2i = p2r;  // edge term (re+, re-, im)
                v4f p1r = p2r, p1n = p2r, p1i = p2r;                   // in-chunk term
                if (kind == 0) {
                    // conj(gx) = M^T gy + e_end (B G)
                    mma_steps<kCC>(0, 16, [&](int k) {
                        const int n = 4 * k + g4;
                        return v4f{sBre[arow * LD + n], sBim[arow * LD + n], sGre[n * SL + bcol],
                                   sGim[n * SL + bcol]};
                    }, p2r, p2n, p2i);
                    // x is real: grad x is the real part, and this term enters neither
                    // the imaginary part nor the row dot product
                    mma_steps<kRR>(rt * 4, R / 4, [&](int k) {
                        const int l = 4 * k + g4;
                        return v4f{sMre[l * RL + arow], 0.f, sGy[l * LD + bcol], 0.f};
                    }, p1r, p1n, p1i);
                } else if (kind == 1) {
                    // conj(gB) = V^T C + e_end (x G^T); x is real
                    mma_steps<kRC>(0, 16, [&](int k) {
                        const int d = 4 * k + g4;
                        return v4f{sXre[arow * LD + d], 0.f, sGre[bcol * SL + d], sGim[bcol * SL + d]};
                    }, p2r, p2n, p2i);
                    mma_steps<kCC>(rt * 4, R / 4, [&](int k) {
                        const int l = 4 * k + g4;
                        return v4f{sVre[l * RL + arow], sVim[l * RL + arow], sCre[l * LD + bcol],
                                   sCim[l * LD + bcol]};
                    }, p1r, p1n, p1i);
                } else {
                    // conj(gC) = V B + e_in (gy H^T)
                    mma_steps<kRC>(0, 16, [&](int k) {
                        const int d = 4 * k + g4;
                        return v4f{sGy[arow * LD + d], 0.f, sHre[bcol * SL + d], sHim[bcol * SL + d]};
                    }, p2r, p2n, p2i);
                    mma_steps<kCC>(0, rt * 4 + 4, [&](int k) {
                        const int sx = 4 * k + g4;
                        return v4f{sVre[arow * RL + sx], sVim[arow * RL + sx], sBre[sx * LD + bcol],
                                   sBim[sx * LD + bcol]};
                    }, p1r, p1n, p1i);
                }
                const int col = ct * 16 + (lane & 15);
                const float *fac = kind == 2 ? sEin : sEend;
                const float *qre = kind == 0 ? sXre : (kind == 1 ? sBre : sCre);
                const float *qim = kind == 0 ? sXim : (kind == 1 ? sBim : sCim);
                // the diagonal pair's term of gB (V[s][s] C_s) and gC (V[l][l] B_l)
                const float *ore = kind == 1 ? sCre : sBre;
                const float *oim = kind == 1 ? sCim : sBim;
                v4f outr, outi, dr, di;
                for (int r = 0; r < 4; ++r) {
                    const int row = rt * 16 + 4 * (lane >> 4) + r;
                    const v2f f = *(const v2f *)&fac[2 * row];
                    const v2f e2 = cmul(f, v2f{p2r[r] - p2n[r], p2i[r]});
                    const v2f e1 = v2f{p1r[r] - p1n[r], p1i[r]};
                    const v2f vd = kind == 0 ? v2f{0.f, 0.f} : *(const v2f *)&sVd[2 * row];
                    const v2f e0 = cmul(vd, v2f{ore[row * LD + col], oim[row * LD + col]});
                    const v2f m = kind == 0 ? e2 : (kind == 1 ? e1 : v2f{e1.x + e2.x, e1.y + e2.y});
                    outr[r] = (e1.x + e2.x) + e0.x;
                    outi[r] = (e1.y + e2.y) + e0.y;
                    const v2f q = v2f{qre[row * LD + col], qim[row * LD + col]};
                    const v2f d = cmul(q, m);
                    dr[r] = d.x;
                    di[r] = d.y;
                }
                dr = row_total(dr);
                di = row_total(di);
                if ((lane & 15) == 15) {
                    const int q = 2 - kind;
                    for (int r = 0; r < 4; ++r) {
                        const int row = rt * 16 + 4 * (lane >> 4) + r;
                        sRow[((q * 4 + ct) * R + row) * 2] = dr[r];
                        sRow[((q * 4 + ct) * R + row) * 2 + 1] = di[r];
                    }
                }
                const int width = kind == 0 ? p.D : p.N;
                const int cols = kind == 0 ? cs.dsl : cs.nsl;
                const int gcol = (kind == 0 ? cs.d0 : cs.n0) + col;
                for (int r = 0; r < 4; ++r) {
                    const int row = rt * 16 + 4 * (lane >> 4) + r;
                    const int t = c * p.Q + row;
                    if (row < p.Q && t < p.T && col < cols) {
                        if constexpr (SLICED) {
                            // partial over the other dimension's slices: gx over S, gB and
                            // gC over T, complex in the (B, T, H, width) layout
                            const int sl = kind == 0 ? cs.st / p.ndb : cs.st % p.ndb;
                            float *part = kind == 0 ? p.gx_part : (kind == 1 ? p.gB_part : p.gC_part);
                            const int64_t g = ((int64_t)b * p.T + t) * p.H + h;
                            const int64_t e = ((int64_t)sl * p.B * p.T * p.H + g) * width + gcol;
                            *(v2f *)&part[2 * e] = v2f{outr[r], -outi[r]};
                            continue;
                        }
                        // real x: its gradient is the real part
                        float *dst = kind == 0 ? p.gx : (kind == 1 ? p.gB : p.gC);
                        const int64_t e = bwd_elem<LAYOUT>(p, b, t, h, width, gcol);
                        bwd_row_store<LAYOUT>(dst, e, outr[r]);
                        if (kind != 0)
                            bwd_row_store<LAYOUT>(dst, e + (int64_t)p.H * p.N, -outi[r]);
                    }
                }
            }
        }
        block_sync();

        if constexpr (FUSED) {
            // G <- exp(Lam[R-1]) G + (e_in o C)^T gy, wave w on tiles w and w + 8 of
            // the 4 x 4 grid (as the adjoint pass); after chunk 0 that is the
            // initial-state gradient (stored conjugated back)
            const v2f dec = cexp_diff(sLam[par], R - 1, -1);
            // tiles w and w + 8 share their columns d (and so the gy operand)
            const int dtl = w & 3, nt0 = w >> 2, nt1 = 2 + (w >> 2);
            const int bd = dtl * 16 + (lane & 15);
            const int an0 = nt0 * 16 + (lane & 15), an1 = nt1 * 16 + (lane & 15);
            v4f re0, im0, re1, im1;
            for (int r = 0; r < 4; ++r) {
                const int n0r = nt0 * 16 + 4 * (lane >> 4) + r, n1r = nt1 * 16 + 4 * (lane >> 4) + r;
                const v2f g0 = cmul_fixed(dec, v2f{sGre[n0r * SL + bd], sGim[n0r * SL + bd]});
                const v2f g1 = cmul_fixed(dec, v2f{sGre[n1r * SL + bd], sGim[n1r * SL + bd]});
                re0[r] = g0.x;
                im0[r] = g0.y;
                re1[r] = g1.x;
                im1[r] = g1.y;
            }
#pragma unroll 1
            for (int l0 = 0; l0 < R; l0 += 4) {
                const int l = l0 + (lane >> 4);
                const v2f ein = *(const v2f *)&sEin[2 * l];
                const v2f a0 = cmul_fixed(v2f{sCre[l * LD + an0], sCim[l * LD + an0]}, ein);
                const v2f a1 = cmul_fixed(v2f{sCre[l * LD + an1], sCim[l * LD + an1]}, ein);
                const float g = sGy[l * LD + bd];
                re0 = mfma_16x16x4(a0.x, g, re0);
                im0 = mfma_16x16x4(a0.y, g, im0);
                re1 = mfma_16x16x4(a1.x, g, re1);
                im1 = mfma_16x16x4(a1.y, g, im1);
            }
            for (int r = 0; r < 4; ++r) {
                const int n0r = nt0 * 16 + 4 * (lane >> 4) + r, n1r = nt1 * 16 + 4 * (lane >> 4) + r;
                if (c == 0) {
                    // after the first chunk: the initial-state gradient, conjugated back
                    if (p.ginit && bd < cs.dsl) {
                        const int64_t base = seq * p.N + cs.n0;
                        if (n0r < cs.nsl)
                            *(v2f *)&p.ginit[2 * ((base + n0r) * p.D + cs.d0 + bd)] = v2f{re0[r], -im0[r]};
                        if (n1r < cs.nsl)
                            *(v2f *)&p.ginit[2 * ((base + n1r) * p.D + cs.d0 + bd)] = v2f{re1[r], -im1[r]};
                    }
                } else {
                    sGre[n0r * SL + bd] = re0[r];
                    sGim[n0r * SL + bd] = im0[r];
                    sGre[n1r * SL + bd] = re1[r];
                    sGim[n1r * SL + bd] = im1[r];
                }
            }
        }

        // Decay gradients. Rows j < R (wave 0): v_j = (O + Off - I)_j and the
        // edge share In_j, summed over the four column tiles in order.
        if (tid < R) {
            v2f v = v2f{0.f, 0.f}, e = v2f{0.f, 0.f};
            for (int ct = 0; ct < 4; ++ct) {
                const float *ooff = &sRow[((0 * 4 + ct) * R + tid) * 2];
                const float *in = &sRow[((1 * 4 + ct) * R + tid) * 2];
                const float *ed = &sRow[((2 * 4 + ct) * R + tid) * 2];
                v.x += ooff[0] - in[0];
                v.y += ooff[1] - in[1];
                e.x += ed[0];
                e.y += ed[1];
            }
            *(v2f *)&sEv[2 * tid] = v;
            *(v2f *)&sEe[2 * tid] = e;
        }
        block_sync();
        // the planes are free once the output tiles and the G update are done
        if (has_next)
            stage(npos.c == p.nc - 1, npos);
        block_sync();
        prev = cur;
        has_prev = true;
        par ^= 1;
        if (!has_next)
            break;
        cur = npos;
    }
    if (w == kGradWave)
        decay_grads(prev, par ^ 1);
}

// Sums the slices' partial gradients in slice order and stores them in the output
// layout: element e < B*T*H*(D + 2N + 1) of [gx (D) | gB (N) | gC (N) | gdt].
template <int LAYOUT>
SSD_KERNEL(256) void bwd_slice_sum_kernel(BwdParams p)
{
    const int64_t rows = (int64_t)p.B * p.T * p.H;
    const int64_t per = (int64_t)p.D + 2 * p.N + 1;
    const int64_t n = rows * per;
    const int64_t step = grid_blocks() * 256;
    for (int64_t e = block_id() * 256 + thread_id(); e < n; e += step) {
        const int64_t g = e / per;  // (b, t, h) flat
        int64_t col = e % per;
        const int64_t bt = g / p.H;
        const int b = (int)(bt / p.T), t = (int)(bt % p.T), h = (int)(g % p.H);
        if (col < p.D) {
            v2f acc = v2f{0.f, 0.f};
            for (int s = 0; s < p.nnb; ++s)
                acc += ld_c(p.gx_part, ((int64_t)s * rows + g) * p.D + col);
            if constexpr (LAYOUT != kLayoutC64)
                bwd_row_store<LAYOUT>(p.gx, bwd_elem<LAYOUT>(p, b, t, h, p.D, (int)col), acc.x);
            else
                *(v2f *)&p.gx[2 * (g * p.D + col)] = acc;
            continue;
        }
        col -= p.D;
        if (col < 2 * p.N) {
            const bool isC = col >= p.N;
            const int nc = (int)(isC ? col - p.N : col);
            const float *part = isC ? p.gC_part : p.gB_part;
            float *dst = isC ? p.gC : p.gB;
            v2f acc = v2f{0.f, 0.f};
            for (int s = 0; s < p.ndb; ++s)
                acc += ld_c(part, ((int64_t)s * rows + g) * p.N + nc);
            if constexpr (LAYOUT != kLayoutC64) {
                const int64_t o = bwd_elem<LAYOUT>(p, b, t, h, p.N, nc);
                bwd_row_store<LAYOUT>(dst, o, acc.x);
                bwd_row_store<LAYOUT>(dst, o + (int64_t)p.H * p.N, acc.y);
            } else {
                *(v2f *)&dst[2 * (g * p.N + nc)] = acc;
            }
            continue;
        }
        float acc = 0.f;
        for (int s = 0; s < p.ns; ++s)
            acc += p.gdt_part[(int64_t)s * rows + g];
        bwd_row_store<LAYOUT>(p.gdt, bwd_elem<LAYOUT>(p, b, t, h, 1, 0), acc);
    }
}

// gA[h] = sum over batch rows and chunks of the per-chunk shares: one
// workgroup per head; thread j adds shares j, j + 256, ... in order, then a
// fixed tree over the threads (the result does not depend on timing).
SSD_KERNEL(256) void bwd_reduce_gA_kernel(const float *part, int B, int H, int nc, float *gA)
{
    SSD_LDS float sre[256];
    SSD_LDS float sim[256];
    const int h = (int)block_id();
    const int tid = thread_id();
    const int64_t n = (int64_t)B * nc;
    float sr = 0.f, si = 0.f;
    for (int64_t k = tid; k < n; k += 256) {
        const int64_t b = k / nc, c = k % nc;
        const v2f v = ld_c(part, (b * H + h) * nc + c);
        sr += v.x;
        si += v.y;
    }
    sre[tid] = sr;
    sim[tid] = si;
    block_sync();
    for (int half = 128; half > 0; half >>= 1) {
        if (tid < half) {
            sre[tid] += sre[tid + half];
            sim[tid] += sim[tid + half];
        }
        block_sync();
    }
    if (tid == 0)
        *(v2f *)&gA[2 * h] = v2f{sre[0], sim[0]};
}

}  // namespace ssd
