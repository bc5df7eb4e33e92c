// Bounds check of the scan kernels under AddressSanitizer on the host
// (TEST INFRASTRUCTURE). Every buffer is an exact-size heap allocation, so any
// read or write past a tensor, or past a shared-memory array, aborts the run.
#include "../../complex_chunkwise_ssd_amd/csrc/ssd_api.hip"

#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <vector>

static float *alloc_fill(size_t n, unsigned &seed)
{
    float *p = (float *)malloc(n * sizeof(float) + (n == 0));
    for (size_t i = 0; i < n; ++i) {
        seed = seed * 1664525u + 1013904223u;
        p[i] = ((seed >> 8) * (1.0f / 16777216.0f) - 0.5f);
    }
    return p;
}

static int run(int B, int T, int H, int N, int D, int Q, bool init, bool fin)
{
    unsigned seed = 12345u + B * 7 + T * 13 + H * 17 + N * 19 + D * 23 + Q * 29;
    float *x = alloc_fill((size_t)B * T * H * D * 2, seed);
    float *A = alloc_fill((size_t)H * 2, seed);
    for (int h = 0; h < H; ++h)
        A[2 * h] = -0.05f - 2.9f * (A[2 * h] + 0.5f);
    float *Bt = alloc_fill((size_t)B * T * H * N * 2, seed);
    float *Ct = alloc_fill((size_t)B * T * H * N * 2, seed);
    float *dt = alloc_fill((size_t)B * T * H, seed);
    float *is = init ? alloc_fill((size_t)B * H * N * D * 2, seed) : nullptr;
    float *y = (float *)malloc(((size_t)B * T * H * D + 1) * sizeof(float));
    float *fs = fin ? (float *)malloc((size_t)B * H * N * D * 2 * sizeof(float)) : nullptr;
    size_t ws = ssd_chunk_forward_workspace_bytes(B, T, H, N, D, Q);
    void *w = ws ? aligned_alloc(256, ws) : nullptr;
    int st = ssd_chunk_forward((ssd_c64 *)x, (ssd_c64 *)A, (ssd_c64 *)Bt, (ssd_c64 *)Ct, dt, B, T, H,
                               N, D, Q, (ssd_c64 *)is, y, (ssd_c64 *)fs, w, ws, nullptr);
    int bad = 0;
    for (size_t i = 0; i < (size_t)B * T * H * D; ++i)
        bad += !isfinite(y[i]);
    printf("B=%d T=%d H=%d N=%d D=%d Q=%d ws=%zu status=%d nonfinite=%d\n", B, T, H, N, D, Q, ws,
           st, bad);
    free(x); free(A); free(Bt); free(Ct); free(dt); free(is); free(y); free(fs); free(w);
    return st != 0 || bad != 0;
}

static int run_bwd(int B, int T, int H, int N, int D, int Q, bool init, bool fin, bool ginit)
{
    unsigned seed = 777u + B * 7 + T * 13 + H * 17 + N * 19 + D * 23 + Q * 29;
    float *x = alloc_fill((size_t)B * T * H * D * 2, seed);
    float *A = alloc_fill((size_t)H * 2, seed);
    for (int h = 0; h < H; ++h)
        A[2 * h] = -0.05f - 2.9f * (A[2 * h] + 0.5f);
    float *Bt = alloc_fill((size_t)B * T * H * N * 2, seed);
    float *Ct = alloc_fill((size_t)B * T * H * N * 2, seed);
    float *dt = alloc_fill((size_t)B * T * H, seed);
    float *gy = alloc_fill((size_t)B * T * H * D, seed);
    float *is = init ? alloc_fill((size_t)B * H * N * D * 2, seed) : nullptr;
    float *gf = fin ? alloc_fill((size_t)B * H * N * D * 2, seed) : nullptr;
    float *gx = (float *)malloc((size_t)B * T * H * D * 2 * sizeof(float) + 1);
    float *gA = (float *)malloc((size_t)H * 2 * sizeof(float));
    float *gB = (float *)malloc((size_t)B * T * H * N * 2 * sizeof(float) + 1);
    float *gC = (float *)malloc((size_t)B * T * H * N * 2 * sizeof(float) + 1);
    float *gdt = (float *)malloc((size_t)B * T * H * sizeof(float) + 1);
    float *gi = ginit ? (float *)malloc((size_t)B * H * N * D * 2 * sizeof(float)) : nullptr;
    size_t ws = ssd_chunk_backward_workspace_bytes(B, T, H, N, D, Q);
    void *w = ws ? aligned_alloc(256, ws) : nullptr;
    int st = ssd_chunk_backward((ssd_c64 *)x, (ssd_c64 *)A, (ssd_c64 *)Bt, (ssd_c64 *)Ct, dt, B, T,
                                H, N, D, Q, (ssd_c64 *)is, gy, (ssd_c64 *)gf, (ssd_c64 *)gx,
                                (ssd_c64 *)gA, (ssd_c64 *)gB, (ssd_c64 *)gC, gdt, (ssd_c64 *)gi, w,
                                ws, nullptr);
    int bad = 0;
    for (size_t i = 0; i < (size_t)B * T * H * D * 2; ++i)
        bad += !isfinite(gx[i]);
    for (size_t i = 0; i < (size_t)B * T * H * N * 2; ++i)
        bad += !isfinite(gB[i]) + !isfinite(gC[i]);
    for (size_t i = 0; i < (size_t)B * T * H; ++i)
        bad += !isfinite(gdt[i]);
    printf("backward B=%d T=%d H=%d N=%d D=%d Q=%d ws=%zu status=%d nonfinite=%d\n", B, T, H, N, D,
           Q, ws, st, bad);
    free(x); free(A); free(Bt); free(Ct); free(dt); free(gy); free(is); free(gf);
    free(gx); free(gA); free(gB); free(gC); free(gdt); free(gi); free(w);
    return st != 0 || bad != 0;
}

static int run_proj(int B, int T, int H, int N, int D, int Q, int extra)
{
    unsigned seed = 999u + B * 7 + T * 13 + H * 17 + N * 19 + D * 23 + Q * 29;
    const int64_t S = (int64_t)H * (D + 4 * N + 1) + extra;
    float *proj = alloc_fill((size_t)B * T * S, seed);
    float *A = alloc_fill((size_t)H * 2, seed);
    for (int h = 0; h < H; ++h)
        A[2 * h] = -0.05f - 2.9f * (A[2 * h] + 0.5f);
    float *y = (float *)malloc(((size_t)B * T * H * D + 1) * sizeof(float));
    float *fs = (float *)malloc((size_t)B * H * N * D * 2 * sizeof(float));
    size_t ws = ssd_chunk_forward_workspace_bytes(B, T, H, N, D, Q);
    void *w = ws ? aligned_alloc(256, ws) : nullptr;
    int st = ssd_chunk_forward_proj(proj, S, (ssd_c64 *)A, B, T, H, N, D, Q, nullptr, y,
                                    (ssd_c64 *)fs, w, ws, nullptr);
    int bad = 0;
    for (size_t i = 0; i < (size_t)B * T * H * D; ++i)
        bad += !isfinite(y[i]);
    printf("proj B=%d T=%d H=%d N=%d D=%d Q=%d ws=%zu status=%d nonfinite=%d\n", B, T, H, N, D, Q,
           ws, st, bad);
    free(proj); free(A); free(y); free(fs); free(w);
    return st != 0 || bad != 0;
}

static int run_bwd_proj(int B, int T, int H, int N, int D, int Q, int extra)
{
    unsigned seed = 4242u + B * 7 + T * 13 + H * 17 + N * 19 + D * 23 + Q * 29;
    const int64_t S = (int64_t)H * (D + 4 * N + 1) + extra;
    float *proj = alloc_fill((size_t)B * T * S, seed);
    float *A = alloc_fill((size_t)H * 2, seed);
    for (int h = 0; h < H; ++h)
        A[2 * h] = -0.05f - 2.9f * (A[2 * h] + 0.5f);
    float *gy = alloc_fill((size_t)B * T * H * D, seed);
    float *gp = (float *)malloc((size_t)B * T * S * sizeof(float));
    for (size_t i = 0; i < (size_t)B * T * S; ++i)
        gp[i] = 0.f;
    float *gA = (float *)malloc((size_t)H * 2 * sizeof(float));
    size_t ws = ssd_chunk_backward_workspace_bytes(B, T, H, N, D, Q);
    void *w = ws ? aligned_alloc(256, ws) : nullptr;
    int st = ssd_chunk_backward_proj(proj, S, (ssd_c64 *)A, B, T, H, N, D, Q, nullptr, gy, nullptr,
                                     gp, (ssd_c64 *)gA, nullptr, w, ws, nullptr);
    int bad = 0;
    for (size_t i = 0; i < (size_t)B * T * S; ++i)
        bad += !isfinite(gp[i]);
    printf("backward proj B=%d T=%d H=%d N=%d D=%d Q=%d ws=%zu status=%d nonfinite=%d\n", B, T, H,
           N, D, Q, ws, st, bad);
    free(proj); free(A); free(gy); free(gp); free(gA); free(w);
    return st != 0 || bad != 0;
}

static int run_bwd_proj_bf16(int B, int T, int H, int N, int D, int Q, int extra)
{
    unsigned seed = 5151u + B * 7 + T * 13 + H * 17 + N * 19 + D * 23 + Q * 29;
    const int64_t S = (int64_t)H * (D + 4 * N + 1) + extra;
    float *src = alloc_fill((size_t)B * T * S, seed);
    uint16_t *proj = (uint16_t *)malloc((size_t)B * T * S * sizeof(uint16_t));
    for (size_t i = 0; i < (size_t)B * T * S; ++i) {
        uint32_t u;
        memcpy(&u, &src[i], 4);
        proj[i] = (uint16_t)(u >> 16);
    }
    float *A = alloc_fill((size_t)H * 2, seed);
    for (int h = 0; h < H; ++h)
        A[2 * h] = -0.05f - 2.9f * (A[2 * h] + 0.5f);
    float *gy = alloc_fill((size_t)B * T * H * D, seed);
    uint16_t *gp = (uint16_t *)calloc((size_t)B * T * S, sizeof(uint16_t));
    float *gA = (float *)malloc((size_t)H * 2 * sizeof(float));
    size_t ws = ssd_chunk_backward_workspace_bytes(B, T, H, N, D, Q);
    void *w = ws ? aligned_alloc(256, ws) : nullptr;
    int st = ssd_chunk_backward_proj_bf16(proj, S, (ssd_c64 *)A, B, T, H, N, D, Q, nullptr, gy,
                                          nullptr, gp, (ssd_c64 *)gA, nullptr, w, ws, nullptr);
    int bad = 0;
    for (size_t i = 0; i < (size_t)B * T * S; ++i)
        bad += (gp[i] & 0x7f80u) == 0x7f80u;  // Inf or NaN
    printf("backward proj bf16 B=%d T=%d H=%d N=%d D=%d Q=%d ws=%zu status=%d nonfinite=%d\n", B,
           T, H, N, D, Q, ws, st, bad);
    free(src); free(proj); free(A); free(gy); free(gp); free(gA); free(w);
    return st != 0 || bad != 0;
}

static int run_mix(int64_t M, int H, int D)
{
    unsigned seed = 31u + (unsigned)M * 7 + H * 17 + D * 23;
    const size_t n = (size_t)M * H * D;
    float *y = alloc_fill(n, seed);
    const size_t F = (size_t)H * D;
    float *W = alloc_fill(F * F, seed);
    float *gz = alloc_fill(n, seed);
    float *z = (float *)malloc(n * sizeof(float) + (n == 0));
    float *gy = (float *)malloc(n * sizeof(float) + (n == 0));
    float *gW = (float *)malloc(F * F * sizeof(float));
    size_t ws = ssd_head_mix_backward_workspace_bytes(M, H, D);
    void *w = ws ? aligned_alloc(256, ws) : nullptr;
    int st = ssd_head_mix(y, W, M, H, D, z, nullptr);
    int st2 = ssd_head_mix_backward(y, W, gz, M, H, D, gy, gW, w, ws, nullptr);
    int bad = 0;
    for (size_t i = 0; i < n; ++i)
        bad += !isfinite(z[i]) + !isfinite(gy[i]);
    for (size_t i = 0; i < F * F; ++i)
        bad += !isfinite(gW[i]);
    printf("mix M=%lld H=%d D=%d ws=%zu status=%d,%d nonfinite=%d\n", (long long)M, H, D, ws, st,
           st2, bad);
    free(y); free(W); free(gz); free(z); free(gy); free(gW); free(w);
    return st != 0 || st2 != 0 || bad != 0;
}

// With the argument "races": a subset for the ThreadSanitizer build (each kind of
// kernel and every barrier pattern once, small enough for the sanitizer's cost).
static int races()
{
    setvbuf(stdout, nullptr, _IOLBF, 0);
    int fails = 0;
    fails += run(16, 20, 16, 4, 6, 16, true, true);   // two chunks per workgroup, staged ahead
    fails += run(1, 130, 1, 8, 8, 3, true, true);     // many segments: prefix and fix-up
    fails += run(1, 40, 1, 130, 70, 16, true, true);  // N and D slices, segments
    fails += run_bwd(16, 37, 16, 4, 6, 32, true, true, true);   // the fused adjoint walk
    fails += run_bwd(1, 70, 1, 64, 64, 64, false, true, true);  // three passes, R = 32
    fails += run_bwd(1, 40, 1, 130, 70, 16, true, true, true);  // state blocks, partials summed
    fails += run_bwd_proj(16, 37, 16, 4, 6, 32, 1);             // the fused walk from in_proj rows
    fails += run_mix(300, 4, 80);   // ragged GEMM tiles, two LDS stages
    fails += run_mix(2100, 2, 4);   // split grad_W and its sum
    printf("%s\n", fails ? "FAIL" : "OK");
    return fails;
}

// With the argument "part=I/N": cases I, I + N, I + 2N, ... of the list (N processes
// can split it); with no argument, every case.
int main(int argc, char **argv)
{
    if (argc > 1 && strcmp(argv[1], "races") == 0)
        return races();
    int part = 0, parts = 1;
    if (argc > 1 && (sscanf(argv[1], "part=%d/%d", &part, &parts) != 2 || parts < 1 || part < 0 ||
                     part >= parts)) {
        fprintf(stderr, "usage: %s [races | part=I/N]\n", argv[0]);
        return 2;
    }
    int fails = 0, k = 0;
#define run(...) (k++ % parts == part ? run(__VA_ARGS__) : 0)
#define run_bwd(...) (k++ % parts == part ? run_bwd(__VA_ARGS__) : 0)
#define run_proj(...) (k++ % parts == part ? run_proj(__VA_ARGS__) : 0)
#define run_bwd_proj(...) (k++ % parts == part ? run_bwd_proj(__VA_ARGS__) : 0)
#define run_bwd_proj_bf16(...) (k++ % parts == part ? run_bwd_proj_bf16(__VA_ARGS__) : 0)
#define run_mix(...) (k++ % parts == part ? run_mix(__VA_ARGS__) : 0)
    fails += run(1, 40, 2, 4, 5, 16, true, true);    // padded N, D; partial chunk
    fails += run(1, 70, 1, 64, 64, 64, false, true);  // full tiles, partial last chunk
    fails += run(1, 45, 1, 6, 70, 32, true, true);    // two D slices
    fails += run(2, 9, 1, 2, 3, 4, false, false);     // Q < 16, no final state
    fails += run(1, 130, 1, 8, 8, 3, true, true);     // many segments
    fails += run(1, 40, 1, 130, 70, 16, true, true);  // N and D slices, segments
    fails += run(2, 9, 1, 256, 3, 4, false, true);    // the largest N, Q < 16
    fails += run(16, 20, 16, 4, 6, 16, true, true);   // 256 sequences: two chunks per workgroup
    fails += run(16, 100, 16, 4, 6, 64, true, true);  // the same with 64-row blocks, partial last chunk
    fails += run_bwd(1, 40, 2, 4, 5, 16, true, true, true);     // padded N, D; partial chunk
    fails += run_bwd(1, 70, 1, 64, 64, 64, false, true, true);  // full tiles, R = 32
    fails += run_bwd(2, 9, 1, 2, 3, 4, false, false, false);    // R = 16, no optional arrays
    fails += run_bwd(1, 33, 3, 8, 64, 256, true, false, true);  // long chunk as 32-token chunks
    fails += run_bwd(16, 37, 16, 4, 6, 32, true, true, true);   // 256 sequences
    fails += run_bwd(1, 40, 1, 130, 70, 16, true, true, true);  // 3 x 2 state blocks, partials summed
    fails += run_proj(1, 40, 2, 4, 6, 16, 0);    // the last row's dt is the last float read
    fails += run_proj(1, 150, 1, 64, 64, 64, 1); // full tiles, segments (stride made even)
    fails += run_proj(2, 9, 1, 2, 4, 4, 1);      // Q < 16
    fails += run_proj(1, 70, 1, 128, 6, 32, 1);  // two N slices (row length made even)
    fails += run_proj(16, 100, 16, 4, 6, 64, 2); // 256 sequences, two chunks per workgroup
    fails += run_bwd_proj(1, 40, 2, 4, 6, 16, 1);   // gradient rows with a spare float
    fails += run_bwd_proj(1, 70, 1, 64, 64, 64, 0); // full tiles
    fails += run_bwd_proj(16, 37, 16, 4, 6, 32, 1); // 256 sequences: the fused adjoint walk
    fails += run_bwd_proj_bf16(1, 40, 2, 4, 6, 16, 1);  // bfloat16 rows, odd row length
    fails += run_mix(5, 16, 64);    // F = 1024: four column tiles, vector loads
    fails += run_mix(3, 7, 10);     // F = 70: scalar loads, ragged tiles
    fails += run_mix(300, 4, 80);   // two ragged row and column tiles
    fails += run_mix(2100, 2, 4);   // the token sum of gW cut into three splits
    fails += run_mix(0, 4, 8);      // no tokens
    printf("%s\n", fails ? "FAIL" : "OK");
    return fails;
}
