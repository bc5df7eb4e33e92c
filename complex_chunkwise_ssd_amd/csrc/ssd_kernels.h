// ssd_kernels.h -- gfx950 kernels of the complex chunkwise SSD scan.
//
// The method (Mamba-3-Lite pages, "Extending" guide Path A Step 1 and Path B
// Step 2, index.html lab 03): per (batch row b, head h)
//   a_t      = softplus(dt_t) * A_h
//   s_t      = exp(a_t) s_{t-1} + B_t x_t^T,     y_t = Re(C_t^T s_t)
// evaluated chunk by chunk. Inside a chunk of Q tokens with running sums
// Lam[l] = a_0 + ... + a_l (relative to the chunk start):
//   Y_diag[l] = sum_{s<=l} (C_l . B_s) exp(Lam[l] - Lam[s]) x_s     (intra-chunk)
//   Y_off[l]  = exp(Lam[l]) C_l^T H_c                               (state-to-output)
//   H_{c+1}   = exp(Lam[Q-1]) H_c + sum_s exp(Lam[Q-1] - Lam[s]) B_s x_s^T
//
// scan_kernel runs one workgroup (eight wave64s) per (b, h, segment, 64-wide
// slice of D) and walks its chunks in order, so the N x 64 state H never
// leaves registers. Every contraction is a real-split fp32 MFMA 16x16x4:
//   G^T = B C^T (complex, K = N)      tile rows s, columns l
//   M   = G o L                       elementwise on the accumulator
//   Y  += Re(M X) + Re(C' H)          M and H feed the next MFMA straight from
//                                     their accumulator layout
//   H   = decay H + B^T (decay' X)    K = chunk rows
// The complex-by-complex products (G and the state update) take three real
// MFMAs per complex product (Gauss's form) instead of four; the products whose
// real part alone is needed take two. The exponents of L are formed from
// running sums restarted on each 16-row tile, so no difference of two long
// running sums is ever taken.
#pragma once

#include <ssd_device.h>
#include <ssd_plan.h>

#include <type_traits>

namespace ssd {

SSD_DEVICE float softplus_f(float v) { return fmaxf(v, 0.f) + log1pf(expf(-fabsf(v))); }

// The same through the hardware's base-2 exponential and logarithm (v_exp_f32,
// v_log_f32, about 1 ulp each): exp(u) = 2^(u log2 e), log(1 + e) = log2(1 + e) ln 2.
// Absolute error below 2e-7 for every v; used where the scan kernel forms its
// decays, whose exponents are later summed over at most a chunk.
SSD_DEVICE float softplus_fast(float v)
{
    const float e = hw_exp2(-fabsf(v) * 1.44269504f);
    return fmaxf(v, 0.f) + hw_log2(1.f + e) * 0.693147181f;
}

SSD_DEVICE v2f cmul(v2f a, v2f b) { return v2f{a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x}; }

// sin and cos by Cody and Waite's additive range reduction (x - k pi/2 with pi/2
// split into three float parts, each step one fused multiply-add) followed by
// the Taylor series of sin and cos on |r| <= pi/4, truncated after r^9 and r^10
// (truncation error below 2e-9). Absolute error about 7e-8 for |x| up to 1e5,
// far beyond the phases the scan produces.
SSD_DEVICE void sincos_cw(float x, float *sp, float *cp)
{
    const float k = rintf(x * 0x1.45f306p-1f);  // nearest multiple of pi/2
    float r = fmaf(-k, 0x1.921fb6p+0f, x);
    r = fmaf(-k, -0x1.777a5cp-25f, r);
    r = fmaf(-k, -0x1.ee59dap-50f, r);
    const float r2 = r * r;
    float ps = fmaf(r2, 0x1.71de3ap-19f, -0x1.a01a02p-13f);  // 1/9!, -1/7!
    ps = fmaf(r2, ps, 0x1.111112p-7f);                       // 1/5!
    ps = fmaf(r2, ps, -0x1.555556p-3f);                      // -1/3!
    const float s = fmaf(r * r2, ps, r);
    float pc = fmaf(r2, -0x1.27e4fcp-22f, 0x1.a01a02p-16f);  // -1/10!, 1/8!
    pc = fmaf(r2, pc, -0x1.6c16c2p-10f);                     // -1/6!
    pc = fmaf(r2, pc, 0x1.555556p-5f);                       // 1/4!
    pc = fmaf(r2, pc, -0.5f);                                // -1/2!
    const float c = fmaf(r2, pc, 1.0f);
    const int q = (int)k;
    const float sv = (q & 1) ? c : s, cv = (q & 1) ? s : c;
    *sp = (q & 2) ? -sv : sv;
    *cp = ((q + 1) & 2) ? -cv : cv;
}

// bfloat16 -> float32: the 16 bits are the high half of the float.
SSD_DEVICE float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
SSD_DEVICE float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

SSD_DEVICE v2f cexp_f(v2f z)
{
    float s, c;
    sincos_cw(z.y, &s, &c);
    const float m = expf(z.x);
    return v2f{m * c, m * s};
}

// exp(z) with the modulus from v_exp_f32 (relative error about 1 ulp plus
// |Re z| 2^-24 from rounding Re z log2 e: under 4e-6 wherever e^{Re z} is a
// normal float). The scan kernel's decays and factors.
SSD_DEVICE v2f cexp_fast(v2f z)
{
    float s, c;
    sincos_cw(z.y, &s, &c);
    const float m = hw_exp2(z.x * 1.44269504f);
    return v2f{m * c, m * s};
}

// ------------------------------------------------------------ discretisation

// A_bar[i] = exp(softplus(dt[i]) * A[i % H]) over the flattened (batch, T, H).
SSD_KERNEL(256) void discretise_abar_kernel(const float *dt, const float *A, int64_t n, int H,
                                            float *abar)
{
    const int64_t i = block_id() * 256 + thread_id();
    if (i >= n)
        return;
    const int h = (int)(i % H);
    const float sp = softplus_f(dt[i]);
    const v2f a = v2f{A[2 * h] * sp, A[2 * h + 1] * sp};
    *(v2f *)&abar[2 * i] = cexp_f(a);
}

// Lambda[b, h, c, l] = sum_{j<=l} softplus(dt[b, cQ+j, h]) * A[h]; one thread
// per (b, c, h), h fastest so that the dt reads of a wave are contiguous.
SSD_KERNEL(256) void discretise_cumsum_kernel(const float *dt, const float *A, int B, int T, int H,
                                              int Q, int nc, float *lam)
{
    const int64_t i = block_id() * 256 + thread_id();
    if (i >= (int64_t)B * nc * H)
        return;
    const int h = (int)(i % H);
    const int c = (int)((i / H) % nc);
    const int b = (int)(i / ((int64_t)H * nc));
    const v2f Ah = v2f{A[2 * h], A[2 * h + 1]};
    v2f run = v2f{0.f, 0.f};
    float *out = lam + (((int64_t)b * H + h) * nc + c) * (int64_t)Q * 2;
    for (int l = 0; l < Q; ++l) {
        const int t = c * Q + l;
        if (t < T) {
            const float sp = softplus_f(dt[((int64_t)b * T + t) * H + h]);
            run.x += sp * Ah.x;
            run.y += sp * Ah.y;
        }
        *(v2f *)&out[2 * l] = run;
    }
}

// final_state = initial_state (or zero) for T == 0.
SSD_KERNEL(256) void copy_state_kernel(const float *src, float *dst, int64_t n)
{
    const int64_t i = block_id() * 256 + thread_id();
    if (i < n)
        dst[i] = src ? src[i] : 0.f;
}

// ------------------------------------------------------------------ the scan

// Calls f(std::integral_constant<int, i>) for i = B .. E-1 (compile-time loop).
template <int B, int E, class F>
SSD_DEVICE void static_for(F &&f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// Causal 16x16 tile pair (st <= lt) of tile index k: the nr diagonal tiles
// first, then the strictly lower ones by increasing lt.
constexpr int tile_lt(int k, int nr)
{
    if (k < nr)
        return k;
    int idx = k - nr, lt = 1;
    while (idx >= lt) {
        idx -= lt;
        ++lt;
    }
    return lt;
}
constexpr int tile_st(int k, int nr)
{
    if (k < nr)
        return k;
    int idx = k - nr, lt = 1;
    while (idx >= lt) {
        idx -= lt;
        ++lt;
    }
    return idx;
}

// R: chunk rows held on chip (chunk_size rounded up to 16, 32 or 64; extra
// rows are identity padding). One segment of one sequence per workgroup: y for
// its tokens and its end state (the final state when there is one segment).
// LAYOUT kLayoutC64: x, B_t, C_t complex64 (B, T, H, .), dt float32 (B, T, H).
// kLayoutProj / kLayoutProjBf16: the inputs are read from an in_proj output row
// per token, [x (H*D, real) | Re B | Im B | Re C | Im C (H*N each) | dt (H)],
// p.tok_stride elements apart, float32 or bfloat16 (widened to float32 as they
// are loaded; all arithmetic stays float32): x is real, so Re(M X) needs only
// Re M and the state update only (decay o B)^T x (half the MFMAs of the
// complex-x steps).
//
// Per chunk c (two barriers, after phase 1 and after phase 2):
//   stage   x moves into the registers phase 1 reads (its B_t and C_t rows and
//           C' = exp(Lam) C, stored as (re, -im), went into LDS during chunk c-1's
//           phase 2, before its closing barrier, so no barrier is needed here).
//   phase 1 (a) M = (B C^T)^T o L^T on the causal tiles (stored as (re, -im)),
//           (b) Re(C' H), (c) H = exp(sum a) H + B^T (decay' o x); wave 0 then
//           forms chunk c+1's per-tile running sums from its dt (already loaded)
//           and the factors exp(Lam) of its C' rows.
//   phase 2 Re(M X); behind its first tile of MFMAs chunk c+1's C_t rows and C'
//           go into LDS, behind its second all threads evaluate chunk c+1's decay
//           factors, at most one complex exponential each; at its end chunk c+1's
//           B_t rows go in (phase 1 of chunk c has finished reading all of these).
//   store   the two waves sharing a column tile combine their partial y.
//
// L on a diagonal 16x16 tile: each lane holds four consecutive s of one row l;
// it takes exp(Lam[l] - Lam[s]) once at the largest causal s of its four and
// walks down with L[l, s] = L[l, s+1] exp(a_{s+1}). Off the diagonal:
// L[l, s] = W[l] K(st, lt) V[s] with W the decay from the start of l's tile,
// V the decay from s to the end of its tile and K the whole tiles in between.
template <int R, int LAYOUT>
SSD_KERNEL(kThreads) void scan_kernel(ScanParams p)
{
    constexpr bool PROJ = LAYOUT != kLayoutC64;
    constexpr bool BF16 = LAYOUT == kLayoutProjBf16;
    constexpr uint32_t ES = BF16 ? 2u : 4u;  // bytes per element of an in_proj row
    constexpr int NR = R / 16;               // 16-row tiles per chunk
    constexpr int NT = NR * (NR + 1) / 2;    // causal tile pairs
    constexpr int NWHOLE = NT < 8 ? NT : 8;  // tiles k < NWHOLE: produced whole by wave k
    constexpr int NSPLIT = NT - NWHOLE;      // the rest: two K halves, waves 2i and 2i+1
    static_assert(NSPLIT == 0 || NSPLIT == 2, "unsupported tile count");
    constexpr int LDI = 2 * kNPad + 4;       // row stride (floats) of an interleaved plane
    constexpr int LOADS = R * (kNPad / 2) / kThreads;  // 16-byte loads per thread per B or C tile
    static_assert(LOADS >= 1, "tile too small for the thread count");
    constexpr uint32_t kOut = 0x80000000u;   // a byte offset past every buffer
    // The wave that scans each chunk's log-decay: below 64 rows (three or one M
    // tiles, on waves 0-2) wave 3, whose SIMD carries no M tile; with ten tiles every
    // SIMD carries two and a half, and wave 0 measured fastest.
    constexpr int kScanWave = NT < 4 ? 3 : 0;

    SSD_LDS float sB[R * LDI];                // B[s][n] interleaved (re, im)
    SSD_LDS float sC[R * LDI];                // C[l][n]
    SSD_LDS float sP[R * LDI];                // exp(Lam[l]) C[l][n] as (re, -im)
    // M tiles (re, -im), lane-major; slots NT .. NT + NSPLIT - 1 hold the second K
    // halves of the tiles k >= NWHOLE (their first halves sit in slot k)
    SSD_LDS v4f sMre[(NT + NSPLIT) * 64], sMim[(NT + NSPLIT) * 64];
    SSD_LDS v4f sYx[4 * NR * 64];             // partial-y exchange
    SSD_LDS v4f sLdre[NR * 64], sLdim[NR * 64];  // L on diagonal tiles, lane-major
    SSD_LDS v2f sDout[R];      // exp(sum of a over rows s+1 .. chunk end)
    SSD_LDS v2f sW[R];         // exp(sum of a over rows tile start .. l)
    SSD_LDS v2f sV[R];         // exp(sum of a over rows s+1 .. end of its tile)
    SSD_LDS v2f sK[NR * NR];   // [st * NR + lt]: exp(sum of a over the tiles strictly between);
                               // [lt * NR + lt]: over the tiles before lt
    SSD_LDS v2f sLam[R];       // running sum of a inside the 16-row tile (inclusive)
    SSD_LDS v2f sSig[R];       // sum of a over rows s+1 .. end of the tile
    SSD_LDS v2f sAbar[R];      // exp(a)
    SSD_LDS v2f sTau[NR + 1];  // tile totals; [NR] = chunk total
    SSD_LDS v2f sDecay[1];     // exp(chunk total)
    SSD_LDS v2f sE[R];         // exp(sum of a over rows 0 .. l): the C' row factors

    const int tid = thread_id();
    const int lane = tid & 63;
    const int w = wave_id();
    const int dtl = w & 3;     // 16-column tile of the D slice
    const int nh = w >> 2;     // half of the state rows (32 of 64)
    const int Lr = lane & 15;
    const int Lk = lane >> 4;

    int64_t blk = block_id();
    const int ns = (int)(blk % p.nnb);  // 64-row slice of the state (N)
    blk /= p.nnb;
    const int db = (int)(blk % p.ndb);
    blk /= p.ndb;
    const int seg = (int)(blk % p.groups_per_seq);
    blk /= p.groups_per_seq;
    const int h = (int)(blk % p.H);
    const int b = (int)(blk / p.H);

    const int64_t row0 = (int64_t)b * p.T * p.H + h;  // flat (b, t=0, h) index
    const int64_t bh = (int64_t)b * p.H + h;
    const v2f Ah = v2f{uniform(p.A[2 * h]), uniform(p.A[2 * h + 1])};
    const uint32_t prow = (uint32_t)p.tok_stride * ES;  // bytes between tokens: in_proj row
    const uint32_t xrow = PROJ ? prow : (uint32_t)(p.H * p.D) * 8u;  //          x
    const uint32_t yrow = (uint32_t)(p.H * p.D) * 4u;                //          y
    const uint32_t brow = PROJ ? prow : (uint32_t)(p.H * p.N) * 8u;  //          B_t, C_t
    const uint32_t drow = PROJ ? prow : (uint32_t)p.H * 4u;          //          dt
    const int64_t bt0 = (int64_t)b * p.T;              // flat (b, t=0) token index
    const int dsl = p.D - db * kDBlock;                // columns of D from this slice on
    const int dl = 16 * dtl + Lr;                      // this lane's column in the slice
    const bool dvalid = dl < dsl;
    const int dcol = db * kDBlock + dl;
    // With N above 64 each workgroup holds 64 state rows, n0 .. n0 + 63: the
    // state update stays within them, and its y (a sum over n) is a partial sum
    // that a later pass adds up over the slices.
    const int n0 = ns * kNPad;
    const int nsl = p.N - n0 < kNPad ? p.N - n0 : kNPad;  // rows of this slice
    float *const yout = p.nnb > 1 ? p.y_part + (int64_t)ns * p.B * p.T * p.H * p.D : p.y;

    // Loop-invariant lane offsets; masked lanes point past the buffer.
    const int ncol = (tid & 31) * 2;
    const uint32_t offB = ncol < nsl ? (uint32_t)(tid >> 5) * brow + ncol * (PROJ ? ES : 8u) : kOut;
    const uint32_t offX = dvalid ? (uint32_t)(4 * Lk) * xrow + dl * (PROJ ? ES : 8u) : kOut;
    const uint32_t offY = dvalid ? (uint32_t)(4 * Lk) * yrow + dl * 4u : kOut;

    // State rows n = 16 * (2 * nh + i) + 4 * Lk + r, column dcol.
    v4f Hre[2], Him[2];
    for (int i = 0; i < 2; ++i) {
        Hre[i] = v4f{0.f, 0.f, 0.f, 0.f};
        Him[i] = v4f{0.f, 0.f, 0.f, 0.f};
    }
    auto add_state = [&](const float *base, v2f scale) {
        // H = scale * H + base[n, dcol] over this lane's elements.
        for (int i = 0; i < 2; ++i)
            for (int r = 0; r < 4; ++r) {
                const int n = 16 * (2 * nh + i) + 4 * Lk + r;
                v2f e = v2f{0.f, 0.f};
                if (n < nsl && dvalid)
                    e = *(const v2f *)&base[((int64_t)(n0 + n) * p.D + dcol) * 2];
                const v2f hv = cmul(scale, v2f{Hre[i][r], Him[i][r]});
                Hre[i][r] = hv.x + e.x;
                Him[i][r] = hv.y + e.y;
            }
    };
    // Segment 0 starts from the initial state, the others from zero (the fix-up
    // pass adds what the state entering them contributes).
    if (seg == 0 && p.init_state)
        add_state(p.init_state + bh * p.N * p.D * 2, v2f{0.f, 0.f});

    const int c_begin = seg * p.spc;
    const int c_end = c_begin + p.spc < p.nc ? c_begin + p.spc : p.nc;
    v2f seg_log = v2f{0.f, 0.f};

    auto rows_of = [&](int c) { return p.Q < p.T - c * p.Q ? p.Q : p.T - c * p.Q; };
    auto tok0 = [&](int c) { return row0 + (int64_t)c * p.Q * p.H; };  // flat (b, cQ, h)
    // PROJ: the first float of chunk c's token row
    auto prow0 = [&](int c) { return (bt0 + (int64_t)c * p.Q) * p.tok_stride; };
    using XT = std::conditional_t<PROJ, float, v2f>;  // x is real in the in_proj layout

    // Registers holding the next chunk's inputs while the current one runs.
    v4f pB[LOADS], pC[LOADS];
    float pdt = 0.f;
    XT pX[NR][4];
    // The next chunk's loads are spread over MFMA steps (a burst of them would hold
    // each wave's in-order issue). Item i < LOADS: a B_t block;
    // then the C_t blocks; then x at (q, j).
    constexpr int NLOAD = 2 * LOADS + 4 * NR;
    buf_t nbB, nbC, nbX;
    // PROJ: one buffer covers both planes of B (and of C); the imaginary plane of a
    // row starts H*N floats after its real plane
    const uint32_t imoff = (uint32_t)(p.H * p.N) * ES;
    // element e of an in_proj row array at base (float32 or bfloat16 elements)
    auto at = [&](const float *base, int64_t e) { return (const void *)((const char *)base + e * ES); };
    // Chunk c's buffers; past the segment's last chunk they are empty, so the loads
    // still issue (keeping the wait counters exact) but read zero.
    auto fetch_begin = [&](int c) {
        if (c < c_end) {
            const uint32_t rows = (uint32_t)rows_of(c);
            if constexpr (PROJ) {
                const int64_t t0 = prow0(c);
                const int64_t hn = (int64_t)h * p.N + n0;
                // rows past the chunk lie past this size (a token row is longer than
                // both planes), so they still read zero
                const uint32_t nb = (rows - 1) * brow + imoff + nsl * ES;
                nbB = make_buf(at(p.Bt, t0 + hn), nb);
                nbC = make_buf(at(p.Ct, t0 + hn), nb);
                nbX = make_buf(at(p.x, t0 + (int64_t)h * p.D + db * kDBlock),
                               (rows - 1) * xrow + dsl * ES);
            } else {
                const int64_t r0 = tok0(c);
                nbB = make_buf(p.Bt + (r0 * p.N + n0) * 2, (rows - 1) * brow + nsl * 8u);
                nbC = make_buf(p.Ct + (r0 * p.N + n0) * 2, (rows - 1) * brow + nsl * 8u);
                nbX = make_buf(p.x + (r0 * p.D + db * kDBlock) * 2, (rows - 1) * xrow + dsl * 8u);
            }
        } else {
            nbB = make_buf(p.Bt, 0u);
            nbC = make_buf(p.Ct, 0u);
            nbX = make_buf(p.x, 0u);
        }
    };
    // Issue order (complex layout): the C_t items, the first KX x items, the B_t
    // items, the other x items; the in_proj layouts keep the storage order.
    constexpr int KX = 2;
    auto fetch_item = [&](auto ic) {
        constexpr int o = decltype(ic)::value;
        constexpr int i = PROJ ? o
                          : o < LOADS       ? LOADS + o
                          : o < LOADS + KX  ? 2 * LOADS + (o - LOADS)
                          : o < 2 * LOADS + KX ? o - LOADS - KX
                                               : o;
        if constexpr (i < LOADS) {
            const uint32_t o = offB + (uint32_t)(16 * i) * brow;
            if constexpr (BF16) {  // two n of the real and of the imaginary plane
                const uint32_t re = buf_load_u32(nbB, o), im = buf_load_u32(nbB, o + imoff);
                pB[i] = v4f{bf16_lo(re), bf16_lo(im), bf16_hi(re), bf16_hi(im)};
            } else if constexpr (PROJ) {
                const v2f re = buf_load2(nbB, o), im = buf_load2(nbB, o + imoff);
                pB[i] = v4f{re.x, im.x, re.y, im.y};
            } else {
                pB[i] = buf_load4(nbB, o);
            }
        } else if constexpr (i < 2 * LOADS) {
            const uint32_t o = offB + (uint32_t)(16 * (i - LOADS)) * brow;
            if constexpr (BF16) {
                const uint32_t re = buf_load_u32(nbC, o), im = buf_load_u32(nbC, o + imoff);
                pC[i - LOADS] = v4f{bf16_lo(re), bf16_lo(im), bf16_hi(re), bf16_hi(im)};
            } else if constexpr (PROJ) {
                const v2f re = buf_load2(nbC, o), im = buf_load2(nbC, o + imoff);
                pC[i - LOADS] = v4f{re.x, im.x, re.y, im.y};
            } else {
                pC[i - LOADS] = buf_load4(nbC, o);
            }
        } else if constexpr (i < NLOAD) {
            constexpr int x = i - 2 * LOADS, q = x >> 2, j = x & 3;
            if constexpr (BF16)
                pX[q][j] = bf16_lo(buf_load_u16(nbX, offX + (uint32_t)(16 * q + j) * xrow));
            else if constexpr (PROJ)
                pX[q][j] = buf_load1(nbX, offX + (uint32_t)(16 * q + j) * xrow);
            else
                pX[q][j] = buf_load2(nbX, offX + (uint32_t)(16 * q + j) * xrow);
        }
    };
    auto fetch = [&](int c) {
        fetch_begin(c);
        static_for<0, NLOAD>([&](auto ic) { fetch_item(ic); });
    };
    // The first NBC items (in issue order) go out with the state steps of phase 1,
    // the rest with the Re(M X) steps of phase 2. Complex layout: the B_t items and
    // two x items (the C_t ones too would outgrow the register budget of the state
    // steps); they then land well before the next stage instead of queuing behind
    // phase 2's MFMAs. In_proj layouts (twice the B_t and C_t load instructions,
    // half the phase 2 MFMAs, real x): all B_t and C_t items.
    constexpr int NBC = PROJ ? 2 * LOADS : LOADS + KX;  // items the state steps issue
    constexpr int PER_S = (NBC + 2 * NR - 1) / (2 * NR);
    // The step logits of chunk c (the scan wave's), loaded a phase ahead of the rest.
    auto fetch_dt = [&](int c) {
        const void *dt0 = PROJ ? at(p.dt, prow0(c) + h) : (const void *)(p.dt + tok0(c));
        const buf_t bT = c < c_end ? make_buf(dt0, (uint32_t)(rows_of(c) - 1) * drow + ES)
                                   : make_buf(p.dt, 0u);
        const uint32_t od = w == kScanWave ? (uint32_t)lane * drow : kOut;
        if constexpr (BF16)
            pdt = bf16_lo(buf_load_u16(bT, od));
        else
            pdt = buf_load1(bT, od);
    };

    // Rows of C_t (and C' = exp(Lam) C_t, stored as (re, -im)) and of B_t into LDS
    // from the prefetch registers.
    auto stage_c = [&]() {
        v2f e[LOADS];
        for (int i = 0; i < LOADS; ++i)
            e[i] = sE[16 * i + (tid >> 5)];
        for (int i = 0; i < LOADS; ++i) {
            const int row = 16 * i + (tid >> 5);
            const v4f vc = pC[i];
            *(v4f *)&sC[row * LDI + 2 * ncol] = vc;
            const v2f c0 = cmul(e[i], v2f{vc.x, vc.y}), c1 = cmul(e[i], v2f{vc.z, vc.w});
            *(v4f *)&sP[row * LDI + 2 * ncol] = v4f{c0.x, -c0.y, c1.x, -c1.y};
        }
    };
    auto stage_b = [&]() {
        for (int i = 0; i < LOADS; ++i)
            *(v4f *)&sB[(16 * i + (tid >> 5)) * LDI + 2 * ncol] = pB[i];
    };

    // The segment's log-decay at each chunk start, for the fix-up pass (one slice of
    // D writes it).
    const buf_t bLog = make_buf(p.chunk_log ? (const void *)(p.chunk_log + bh * p.nc * 2)
                                            : (const void *)p.dt,
                                p.chunk_log && db == 0 && ns == 0 ? (uint32_t)p.nc * 8u : 0u);

    // One wave: running sums of a = softplus(dt) A inside each 16-row tile of chunk c.
    auto scan = [&](int c) {
        const int rows = rows_of(c);
        const float sp = softplus_fast(pdt);
        const v2f a = lane < rows ? v2f{Ah.x * sp, Ah.y * sp} : v2f{0.f, 0.f};
        // inclusive running sums inside the tile, forwards (lam) and backwards (rs)
        v2f lam = a, rs = a;
        lam += v2f{row_shr<1>(lam.x), row_shr<1>(lam.y)};
        rs += v2f{row_shl<1>(rs.x), row_shl<1>(rs.y)};
        lam += v2f{row_shr<2>(lam.x), row_shr<2>(lam.y)};
        rs += v2f{row_shl<2>(rs.x), row_shl<2>(rs.y)};
        lam += v2f{row_shr<4>(lam.x), row_shr<4>(lam.y)};
        rs += v2f{row_shl<4>(rs.x), row_shl<4>(rs.y)};
        lam += v2f{row_shr<8>(lam.x), row_shr<8>(lam.y)};
        rs += v2f{row_shl<8>(rs.x), row_shl<8>(rs.y)};
        const v2f sig = v2f{row_shl<1>(rs.x), row_shl<1>(rs.y)};  // rows s+1 .. tile end
        v2f tau[NR];
        v2f tot = v2f{0.f, 0.f};
        for (int t = 0; t < NR; ++t) {
            tau[t] = v2f{lane_read(lam.x, 16 * t + 15), lane_read(lam.y, 16 * t + 15)};
            tot += tau[t];
        }
        v2f before = v2f{0.f, 0.f};  // the tiles before this lane's
        for (int t = 0; t < NR - 1; ++t)
            if (t < (lane >> 4))
                before += tau[t];
        if (lane < R) {
            sLam[lane] = lam;
            sSig[lane] = sig;
            sAbar[lane] = cexp_fast(a);
            sE[lane] = cexp_fast(lam + before);
        }
        if (lane == 0) {
            for (int t = 0; t < NR; ++t)
                sTau[t] = tau[t];
            sTau[NR] = tot;
        }
        const uint32_t olog = lane == 0 ? (uint32_t)c * 8u : kOut;
        buf_store1(bLog, olog, seg_log.x);
        buf_store1(bLog, olog + 4u, seg_log.y);
        seg_log += tot;
    };

    // All threads: chunk c's decay factors from sLam, sSig, sAbar, sTau, at most one
    // complex exponential per thread. Waves 0-3: diagonal-tile L, one lane-quad each;
    // wave 4: W; wave 5: the tile constants K and the chunk decay; wave 6: the decay
    // to the chunk end; wave 7: V.
    auto factors = [&]() {
        if (tid < 256) {
            if (tid < NR * 64) {
                const int tile = tid >> 6, ln = tid & 63;
                const int l = ln & 15, g = 4 * (ln >> 4);
                const v2f *lam = sLam + 16 * tile;
                v2f L = l >= g + 3 ? cexp_fast(lam[l] - lam[g + 3]) : v2f{0.f, 0.f};
                v4f lre, lim;
                lre[3] = L.x;
                lim[3] = L.y;
                for (int r = 2; r >= 0; --r) {
                    if (l > g + r)
                        L = cmul(L, sAbar[16 * tile + g + r + 1]);
                    else
                        L = l == g + r ? v2f{1.f, 0.f} : v2f{0.f, 0.f};
                    lre[r] = L.x;
                    lim[r] = L.y;
                }
                sLdre[tid] = lre;
                sLdim[tid] = lim;
            }
            return;
        }
        const int role = (tid >> 6) - 4, ri = tid & 63;
        if (role == 0) {
            if (ri < R)
                sW[ri] = cexp_fast(sLam[ri]);
        } else if (role == 1) {
            // K(st, lt), st < lt: the tiles strictly between; K(lt, lt): the tiles before
            // lt; slot NR * NR: the whole chunk (the decay of the state).
            const int st = ri / NR, lt = ri % NR;
            v2f tau[NR];  // read before any branch: one LDS round trip
            for (int t = 0; t < NR; ++t)
                tau[t] = sTau[t];
            if (ri <= NR * NR && (ri == NR * NR || st <= lt)) {
                v2f z = v2f{0.f, 0.f};
                for (int t = 0; t < NR; ++t)
                    if (ri == NR * NR || (st < lt ? (t > st && t < lt) : t < lt))
                        z += tau[t];
                const v2f e = cexp_fast(z);
                if (ri == NR * NR)
                    sDecay[0] = e;
                else
                    sK[ri] = e;
            }
        } else if (role == 2) {
            v2f tau[NR];
            for (int t = 0; t < NR; ++t)
                tau[t] = sTau[t];
            if (ri < R) {
                v2f z = sSig[ri];
                for (int t = 0; t < NR; ++t)
                    if (t > (ri >> 4))
                        z += tau[t];
                sDout[ri] = cexp_fast(z);
            }
        } else {
            if (ri < R)
                sV[ri] = cexp_fast(sSig[ri]);
        }
    };
    static_assert(R <= 64 && NR * NR < 63, "role layout assumes at most 64 rows");

    if (c_begin < c_end) {
        fetch(c_begin);
        fetch_dt(c_begin);
        if (w == kScanWave)
            scan(c_begin);
        block_sync();
        factors();
        stage_c();
        stage_b();
        block_sync();
    }

    for (int c = c_begin; c < c_end; ++c) {
        const int rows = rows_of(c);
        const int64_t r0 = tok0(c);

        // ---- stage: x into the registers phase 1 reads. The chunk's rows are in LDS
        // already (staged in the previous chunk's phase 2 or the prologue, before a
        // barrier), so phase 1 starts without one.
        XT X[NR][4];  // x[s][dcol] with s = 16 q + 4 Lk + j
        for (int q = 0; q < NR; ++q)
            for (int j = 0; j < 4; ++j)
                X[q][j] = pX[q][j];
        const bool more = c + 1 < c_end;
        fetch_dt(c + 1);
        fetch_begin(c + 1);

        v4f Y[NR];
        for (int lt = 0; lt < NR; ++lt)
            Y[lt] = v4f{0.f, 0.f, 0.f, 0.f};
        // ---- phase 1a: M tiles. Whole tiles k < NWHOLE by wave k; the others as
        // two K halves accumulated into LDS (two adds onto zero: order-free).
        {
            auto produce = [&](auto kc, auto q0c, auto q1c) {
                constexpr int k = decltype(kc)::value;
                constexpr int st = tile_st(k, NR), lt = tile_lt(k, NR);
                // G^T[s][l] = sum_n B[s][n] C[l][n] with three real products per
                // complex one (Gauss): P1 = sum Bre Cre, P2 = sum Bim Cim,
                // P3 = sum (Bre + Bim)(Cre + Cim); re = P1 - P2, im = P3 - P1 - P2.
                v4f p1 = v4f{0.f, 0.f, 0.f, 0.f}, p2 = v4f{0.f, 0.f, 0.f, 0.f};
                v4f p3 = v4f{0.f, 0.f, 0.f, 0.f};
                constexpr int Q0 = decltype(q0c)::value, Q1 = decltype(q1c)::value;
                // operand blocks of half-step h (B and C rows, two n each), in flight one
                // half-step ahead
                v4f ob[2][2];
                auto load = [&](int hs, v4f *o) {
                    const int col = 2 * (16 * (hs >> 1) + 4 * Lk + 2 * (hs & 1));
                    o[0] = *(const v4f *)&sB[(16 * st + Lr) * LDI + col];
                    o[1] = *(const v4f *)&sC[(16 * lt + Lr) * LDI + col];
                };
                load(2 * Q0, ob[0]);
                static_for<2 * Q0, 2 * Q1>([&](auto hc) {
                    constexpr int hs = decltype(hc)::value, cur = hs & 1;
                    if constexpr (hs + 1 < 2 * Q1)
                        load(hs + 1, ob[cur ^ 1]);
                    sched_fence();
                    const v4f bb = ob[cur][0], cc = ob[cur][1];
                    const float bre[2] = {bb.x, bb.z}, bim[2] = {bb.y, bb.w};
                    const float cre[2] = {cc.x, cc.z}, cim[2] = {cc.y, cc.w};
                    for (int j = 0; j < 2; ++j) {
                        p1 = mfma_16x16x4(bre[j], cre[j], p1);
                        p2 = mfma_16x16x4(bim[j], cim[j], p2);
                        p3 = mfma_16x16x4(bre[j] + bim[j], cre[j] + cim[j], p3);
                    }
                    sched_fence();
                });
                const v4f gre = p1 - p2, gim = p3 - p1 - p2;
                // Accumulator element r of this lane: s = 16 st + 4 Lk + r, l = 16 lt + Lr.
                v4f mre, mim;
                if constexpr (st == lt) {
                    const v4f lre = sLdre[st * 64 + lane], lim = sLdim[st * 64 + lane];
                    for (int r = 0; r < 4; ++r) {
                        mre[r] = gre[r] * lre[r] - gim[r] * lim[r];
                        mim[r] = -(gre[r] * lim[r] + gim[r] * lre[r]);
                    }
                } else {
                    const v2f wk = cmul(sW[16 * lt + Lr], sK[st * NR + lt]);
                    for (int r = 0; r < 4; ++r) {
                        const v2f L = cmul(wk, sV[16 * st + 4 * Lk + r]);
                        mre[r] = gre[r] * L.x - gim[r] * L.y;
                        mim[r] = -(gre[r] * L.y + gim[r] * L.x);
                    }
                }
                // a split tile's halves go to two slots (plain stores; the consumer adds them)
                constexpr int slot = k < NWHOLE || Q0 == 0 ? k : NT + (k - NWHOLE);
                sMre[slot * 64 + lane] = mre;
                if constexpr (!PROJ)
                    sMim[slot * 64 + lane] = mim;
            };
            using I0 = std::integral_constant<int, 0>;
            using I2 = std::integral_constant<int, 2>;
            using I4 = std::integral_constant<int, kNPad / 16>;
            static_for<0, NT>([&](auto kc) {
                constexpr int k = decltype(kc)::value;
                if constexpr (k < NWHOLE) {
                    if (w == k)
                        produce(kc, I0{}, I4{});
                } else {
                    if (w == 2 * (k - NWHOLE))
                        produce(kc, I0{}, I2{});
                    else if (w == 2 * (k - NWHOLE) + 1)
                        produce(kc, I2{}, I4{});
                }
            });

            // ---- phase 1b: Re(C' H) over this wave's half of the state rows; H is the
            // B operand straight from its accumulator layout.
            {
                v4f oa[2][2];
                auto load = [&](int g, v4f *o) {  // step g = (lt, i)
                    const int lt = g >> 1, i = g & 1;
                    const float *pp = &sP[(16 * lt + Lr) * LDI + 2 * (16 * (2 * nh + i) + 4 * Lk)];
                    o[0] = *(const v4f *)pp;
                    o[1] = *(const v4f *)(pp + 4);
                };
                load(0, oa[0]);
                static_for<0, 2 * NR>([&](auto gc) {
                    constexpr int g = decltype(gc)::value, lt = g >> 1, i = g & 1, cur = g & 1;
                    if constexpr (g + 1 < 2 * NR)
                        load(g + 1, oa[cur ^ 1]);
                    sched_fence();
                    const v4f a01 = oa[cur][0], a23 = oa[cur][1];
                    const float are[4] = {a01.x, a01.z, a23.x, a23.z};
                    const float aim[4] = {a01.y, a01.w, a23.y, a23.w};
                    for (int r = 0; r < 4; ++r) {
                        Y[lt] = mfma_16x16x4(are[r], Hre[i][r], Y[lt]);
                        Y[lt] = mfma_16x16x4(aim[r], Him[i][r], Y[lt]);
                    }
                    sched_fence();
                });
            }
        }

        // ---- phase 1c: H = exp(sum a) H + B^T (decay' o x).
        {
            const v2f g = sDecay[0];
            for (int i = 0; i < 2; ++i)
                for (int r = 0; r < 4; ++r) {
                    const v2f hv = cmul(g, v2f{Hre[i][r], Him[i][r]});
                    Hre[i][r] = hv.x;
                    Him[i][r] = hv.y;
                }
            // operands of group g = (q, i): B at four rows of step q for this wave's state-row
            // tile i, and (with i = 0) the decay of those rows to the chunk end; in flight
            // one group ahead
            v2f ob[2][4], od[2][4];
            auto load = [&](int g, v2f *bb, v2f *d) {
                const int q = g >> 1, i = g & 1;
                for (int j = 0; j < 4; ++j) {
                    const int s = 16 * q + 4 * Lk + j;
                    bb[j] = *(const v2f *)&sB[s * LDI + 2 * (16 * (2 * nh + i) + Lr)];
                    if (i == 0)
                        d[j] = sDout[s];
                }
            };
            load(0, ob[0], od[0]);
            // complex x, three real products per complex one (Gauss): with x' = decay' o x,
            // k1 = (Bre + Bim) x're, k2 = Bim (x're + x'im), k3 = Bre (x'im - x're);
            // the update's re = k1 - k2 and im = k1 + k3, k1 summed apart and added to both
            float xr[4], xn[4], xd[4];
            v4f K1[2];
            for (int i = 0; i < 2; ++i)
                K1[i] = v4f{0.f, 0.f, 0.f, 0.f};
            static_for<0, 2 * NR>([&](auto gc) {
                constexpr int g = decltype(gc)::value, q = g >> 1, i = g & 1, cur = g & 1;
                if constexpr (g + 1 < 2 * NR)
                    load(g + 1, ob[cur ^ 1], od[q & 1 ^ (i == 1 ? 1 : 0)]);
                static_for<g * PER_S, ((g + 1) * PER_S < NBC ? (g + 1) * PER_S : NBC)>(
                    [&](auto ic) { fetch_item(ic); });
                sched_fence();
                if constexpr (PROJ) {
                    // real x: (decay o B) against x, two MFMAs per step
                    for (int j = 0; j < 4; ++j) {
                        const v2f bv = cmul(od[q & 1][j], ob[cur][j]);
                        Hre[i] = mfma_16x16x4(bv.x, X[q][j], Hre[i]);
                        Him[i] = mfma_16x16x4(bv.y, X[q][j], Him[i]);
                    }
                } else {
                    if constexpr (i == 0)
                        for (int j = 0; j < 4; ++j) {
                            const v2f xs = cmul(od[q & 1][j], X[q][j]);
                            xr[j] = xs.x;
                            xn[j] = -xs.x - xs.y;
                            xd[j] = xs.y - xs.x;
                        }
                    for (int j = 0; j < 4; ++j) {
                        const v2f bv = ob[cur][j];
                        K1[i] = mfma_16x16x4(bv.x + bv.y, xr[j], K1[i]);
                        Hre[i] = mfma_16x16x4(bv.y, xn[j], Hre[i]);
                        Him[i] = mfma_16x16x4(bv.x, xd[j], Him[i]);
                    }
                }
                sched_fence();
            });
            if constexpr (!PROJ)
                for (int i = 0; i < 2; ++i) {
                    Hre[i] += K1[i];
                    Him[i] += K1[i];
                }
        }
        if (more && w == kScanWave)
            scan(c + 1);
        block_sync();

        // ---- phase 2: intra-chunk term Re(M X) = Mre Xre + (-Mim) Xim; the tiles of a
        // column tile are split between its two waves by parity. Behind the MFMAs of
        // the first tile, the next chunk's C_t rows and C' (all its rows in the
        // in_proj layouts) go into LDS, which phase 1 has finished reading; behind
        // those of the second, the next chunk's decay factors (phase 2 reads none of
        // the arrays they overwrite), so that their LDS round trips overlap MFMAs.
        {
            constexpr int kStageTile = 0;
            constexpr int kFactorTile = 1;
            auto stage_next = [&]() {
                if (more) {
                    stage_c();
                    if constexpr (PROJ)
                        stage_b();
                }
            };
            auto ydiag = [&](auto nhc) {
                constexpr int NH = decltype(nhc)::value;
                constexpr int NK = (NT + 1 - NH) / 2;  // tiles k = NH, NH + 2, ...
                constexpr int NX = NLOAD - NBC;         // items left for phase 2
                constexpr int NKD = NK > 0 ? NK : 1;     // (no tiles: PER_K unused)
                constexpr int PER_K = NK > 0 ? (NX + NKD - 1) / NKD : 0;
                // M tiles in flight one tile ahead (a split tile: both halves)
                v4f mre[2], mim[2], mre2, mim2;
                auto loadm = [&](auto kc, int b) {
                    constexpr int k = decltype(kc)::value;
                    mre[b] = sMre[k * 64 + lane];
                    if constexpr (!PROJ)
                        mim[b] = sMim[k * 64 + lane];
                    if constexpr (k >= NWHOLE) {
                        mre2 = sMre[(NT + k - NWHOLE) * 64 + lane];
                        if constexpr (!PROJ)
                            mim2 = sMim[(NT + k - NWHOLE) * 64 + lane];
                    }
                };
                if constexpr (NK > 0)
                    loadm(std::integral_constant<int, NH>{}, 0);
                static_for<0, NK>([&](auto ic) {
                    constexpr int i = decltype(ic)::value, k = 2 * i + NH, cur = i & 1;
                    constexpr int st = tile_st(k, NR), lt = tile_lt(k, NR);
                    if constexpr (i + 1 < NK)
                        loadm(std::integral_constant<int, k + 2>{}, cur ^ 1);
                    constexpr int a = NBC + i * PER_K, e = NBC + (i + 1) * PER_K;
                    static_for<a, (e < NLOAD ? e : NLOAD)>([&](auto xc) { fetch_item(xc); });
                    sched_fence();
                    if constexpr (k >= NWHOLE) {
                        mre[cur] += mre2;
                        if constexpr (!PROJ)
                            mim[cur] += mim2;
                    }
                    for (int r = 0; r < 4; ++r) {
                        if constexpr (PROJ) {
                            Y[lt] = mfma_16x16x4(mre[cur][r], X[st][r], Y[lt]);
                        } else {
                            Y[lt] = mfma_16x16x4(mre[cur][r], X[st][r].x, Y[lt]);
                            Y[lt] = mfma_16x16x4(mim[cur][r], X[st][r].y, Y[lt]);
                        }
                    }
                    if constexpr (i == kStageTile)
                        stage_next();
                    if constexpr (i == kFactorTile)
                        if (more)
                            factors();
                    sched_fence();
                });
                if constexpr (NK == 0)
                    static_for<NBC, NLOAD>([&](auto xc) { fetch_item(xc); });
                if constexpr (NK <= kStageTile)
                    stage_next();
                if constexpr (NK <= kFactorTile)
                    if (more)
                        factors();
            };
            if (nh == 0)
                ydiag(std::integral_constant<int, 0>{});
            else
                ydiag(std::integral_constant<int, 1>{});
            // Row tile lt is finished and stored by the wave with nh == lt % 2; each wave
            // hands its partial sums of the other tiles over through LDS.
            for (int j = 0; j < (NR + 1) / 2; ++j) {
                const int lt = 2 * j + 1 - nh;  // a tile this wave does not own
                if (lt < NR)
                    sYx[(dtl * NR + lt) * 64 + lane] = nh ? Y[2 * j] : Y[2 * j + 1 < NR ? 2 * j + 1 : 0];
            }
            if constexpr (!PROJ)
                if (more)
                    stage_b();
        }
        block_sync();

        // ---- store y. Straight-line stores (a tile this wave does not own is aimed
        // past the buffer), so the wait counters stay exact across the loop.
        {
            const buf_t bY = make_buf(yout + r0 * p.D + db * kDBlock,
                                      (uint32_t)(rows - 1) * yrow + dsl * 4u);
            for (int j = 0; j < (NR + 1) / 2; ++j) {
                const int lt = 2 * j + nh;
                const bool own = lt < NR;
                const v4f mine = nh && 2 * j + 1 < NR ? Y[2 * j + 1] : Y[2 * j];
                const v4f o = sYx[(dtl * NR + (own ? lt : 0)) * 64 + lane];
                const uint32_t off = own ? offY + (uint32_t)(16 * lt) * yrow : kOut;
                for (int r = 0; r < 4; ++r)
                    buf_store1(bY, off + (uint32_t)r * yrow, mine[r] + o[r]);
            }
        }
    }

    // ---- results of the segment.
    float *out = nullptr;
    if (p.P == 1) {
        out = p.final_state ? p.final_state + bh * p.N * p.D * 2 : nullptr;
    } else {
        const int64_t sidx = bh * p.P + seg;
        out = p.seg_state + sidx * p.N * p.D * 2;
        if (db == 0 && ns == 0 && tid == kScanWave * 64)  // the scan wave holds the total
            *(v2f *)&p.seg_logdecay[sidx * 2] = seg_log;
    }
    if (out) {
        for (int i = 0; i < 2; ++i)
            for (int r = 0; r < 4; ++r) {
                const int n = 16 * (2 * nh + i) + 4 * Lk + r;
                if (n < nsl && dvalid)
                    *(v2f *)&out[((int64_t)(n0 + n) * p.D + dcol) * 2] = v2f{Hre[i][r], Him[i][r]};
            }
    }
}

}  // namespace ssd
