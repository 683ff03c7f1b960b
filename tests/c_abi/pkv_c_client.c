/* A C consumer of libpkv: built with a plain C compiler (no PyTorch, no HIP
 * compiler), it allocates every buffer with the HIP runtime API and drives
 * the library through include/pkv.h alone (the C ABI of the PersistentKV
 * page's decode engine: create, build the compact queue, decode, destroy).
 *
 * Inputs come from a small integer recipe of this file: values are multiples
 * of 1/8 in [-1, 1] (exact in bf16), the pages of the rows are scattered over
 * the pool by a seeded shuffle, unused pool slots and past-the-end token rows
 * hold NaN, block-table entries past a row's pages hold -1, and one row is
 * empty.  The program writes its host-side inputs and the outputs it read
 * back to a binary file for the test that checks them against the oracle.
 *
 *   pkv_c_client <output file>
 * Exit status 0 on success; any failed call prints the library's reason. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "pkv.h"

enum { B = 4, HQ = 8, HKV = 2, D = 128, P = 16, SPARE = 2 };
static const int32_t LENS[B] = {37, 1000, 0, 5000};

static uint32_t mix(uint32_t x) {            /* integer hash (xorshift-multiply) */
    x ^= x >> 16; x *= 0x7feb352dU; x ^= x >> 15; x *= 0x846ca68bU; x ^= x >> 16;
    return x;
}

static uint16_t value_bits(uint32_t stream, uint32_t i) {   /* (h % 17 - 8) / 8 as bf16 */
    const float v = (float)((int)(mix(i * 2654435761U ^ stream) % 17U) - 8) * 0.125f;
    uint32_t u;
    memcpy(&u, &v, 4);
    return (uint16_t)(u >> 16);               /* exact: at most 4 significant bits */
}

#define CHECK_HIP(call)                                                              \
    do {                                                                             \
        hipError_t e_ = (call);                                                      \
        if (e_ != hipSuccess) { fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_)); return 2; } \
    } while (0)
#define CHECK_PKV(call, h)                                                           \
    do {                                                                             \
        pkv_status s_ = (call);                                                      \
        if (s_ != PKV_OK) {                                                          \
            fprintf(stderr, "%s: %s (%s)\n", #call, pkv_status_string(s_), pkv_last_error(h)); return 3; \
        }                                                                            \
    } while (0)

int main(int argc, char** argv) {
    if (argc != 2) { fprintf(stderr, "usage: pkv_c_client <output file>\n"); return 1; }
    int32_t pages_of[B], max_pages = 1, npg = SPARE;
    for (int b = 0; b < B; ++b) {
        pages_of[b] = (LENS[b] + P - 1) / P;
        npg += pages_of[b];
        if (pages_of[b] > max_pages) max_pages = pages_of[b];
    }
    const size_t pool_elems = (size_t)npg * HKV * P * D;
    const size_t q_elems = (size_t)B * HQ * D;

    /* host inputs */
    int32_t* perm = malloc(sizeof(int32_t) * npg);
    int32_t* bt = malloc(sizeof(int32_t) * B * max_pages);
    uint16_t* q = malloc(2 * q_elems);
    uint16_t* k = malloc(2 * pool_elems);
    uint16_t* v = malloc(2 * pool_elems);
    uint16_t* out = malloc(2 * q_elems);
    float* lse = malloc(sizeof(float) * B * HQ);
    if (!perm || !bt || !q || !k || !v || !out || !lse) { fprintf(stderr, "host allocation failed\n"); return 2; }
    for (int i = 0; i < npg; ++i) perm[i] = i;
    uint32_t st = 12345U;
    for (int i = npg - 1; i > 0; --i) {        /* seeded Fisher-Yates shuffle */
        st = st * 1664525U + 1013904223U;
        const int j = (int)(st % (uint32_t)(i + 1));
        const int32_t t = perm[i]; perm[i] = perm[j]; perm[j] = t;
    }
    for (size_t i = 0; i < q_elems; ++i) q[i] = value_bits(0x51U, (uint32_t)i);
    for (size_t i = 0; i < pool_elems; ++i) { k[i] = 0x7FC0; v[i] = 0x7FC0; }   /* NaN everywhere unused */
    int next = 0;
    for (int b = 0; b < B; ++b)
        for (int j = 0; j < max_pages; ++j) {
            if (j >= pages_of[b]) { bt[b * max_pages + j] = -1; continue; }
            const int32_t pg = perm[next++];
            bt[b * max_pages + j] = pg;
            for (int h = 0; h < HKV; ++h)
                for (int r = 0; r < P; ++r) {
                    if (j * P + r >= LENS[b]) continue;                       /* past the end: NaN */
                    for (int d = 0; d < D; ++d) {
                        const size_t at = (((size_t)pg * HKV + h) * P + r) * D + d;
                        const uint32_t tok = (uint32_t)(((b * 65536 + j * P + r) * HKV + h) * D + d);
                        k[at] = value_bits(0x4BU, tok);
                        v[at] = value_bits(0x56U, tok);
                    }
                }
        }

    /* a configuration the library must refuse, with a reason */
    pkv_config bad;
    memset(&bad, 0, sizeof(bad));
    bad.struct_size = sizeof(pkv_config);
    bad.num_q_heads = HQ; bad.num_kv_heads = HKV; bad.head_dim = 96; bad.page_size = P;
    bad.num_pages = npg; bad.max_batch = B; bad.max_pages_per_seq = max_pages;
    size_t bytes = 0;
    const pkv_status sb = pkv_workspace_size(&bad, &bytes);
    if (sb == PKV_OK) { fprintf(stderr, "head_dim 96 was accepted\n"); return 4; }
    printf("refused head_dim 96: %s\n", pkv_status_string(sb));

    pkv_config cfg = bad;
    cfg.head_dim = D;
    CHECK_PKV(pkv_workspace_size(&cfg, &bytes), NULL);

    void *dq, *dk, *dv, *dbt, *dlens, *dout, *dlse, *ws;
    hipStream_t stream;
    CHECK_HIP(hipStreamCreate(&stream));
    CHECK_HIP(hipMalloc(&dq, 2 * q_elems));
    CHECK_HIP(hipMalloc(&dk, 2 * pool_elems));
    CHECK_HIP(hipMalloc(&dv, 2 * pool_elems));
    CHECK_HIP(hipMalloc(&dbt, sizeof(int32_t) * B * max_pages));
    CHECK_HIP(hipMalloc(&dlens, sizeof(int32_t) * B));
    CHECK_HIP(hipMalloc(&dout, 2 * q_elems));
    CHECK_HIP(hipMalloc(&dlse, sizeof(float) * B * HQ));
    CHECK_HIP(hipMalloc(&ws, bytes));
    CHECK_HIP(hipMemcpy(dq, q, 2 * q_elems, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dk, k, 2 * pool_elems, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dv, v, 2 * pool_elems, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dbt, bt, sizeof(int32_t) * B * max_pages, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dlens, LENS, sizeof(int32_t) * B, hipMemcpyHostToDevice));

    pkv_handle* h = NULL;
    if (pkv_create(&cfg, ws, bytes / 2, stream, &h) == PKV_OK) {             /* too small a workspace */
        fprintf(stderr, "a workspace of half the size was accepted\n");
        return 4;
    }
    CHECK_PKV(pkv_create(&cfg, ws, bytes, stream, &h), NULL);
    pkv_queue_info info;
    CHECK_PKV(pkv_build_queue(h, LENS, B, &info), h);
    pkv_tensors t;
    memset(&t, 0, sizeof(t));
    t.q = dq; t.k_pool = dk; t.v_pool = dv; t.block_table = (const int32_t*)dbt;
    t.ctx_lens = (const int32_t*)dlens; t.out = dout; t.lse = (float*)dlse;
    t.batch = B; t.block_table_stride = max_pages;
    for (int call = 0; call < 2; ++call) CHECK_PKV(pkv_decode(h, &t, stream), h);
    CHECK_HIP(hipStreamSynchronize(stream));
    pkv_runtime_info ri;
    CHECK_PKV(pkv_query(h, &ri), h);
    if (ri.error_code != 0) { fprintf(stderr, "device error word %u\n", ri.error_code); return 5; }
    CHECK_HIP(hipMemcpy(out, dout, 2 * q_elems, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(lse, dlse, sizeof(float) * B * HQ, hipMemcpyDeviceToHost));
    CHECK_PKV(pkv_destroy(h), NULL);
    printf("decoded: %d items, split %d, range %d tokens, %d CUs, %u decode calls\n", info.n_items,
           info.split, info.chunk_tokens, ri.num_cus, ri.decode_calls);

    FILE* f = fopen(argv[1], "wb");
    if (!f) { perror("output file"); return 6; }
    const int32_t hdr[12] = {0x504B5643, B, HQ, HKV, D, P, npg, max_pages,
                             info.n_items, info.split, info.chunk_tokens, ri.num_cus};
    fwrite(hdr, sizeof(hdr), 1, f);
    fwrite(LENS, sizeof(int32_t), B, f);
    fwrite(bt, sizeof(int32_t), (size_t)B * max_pages, f);
    fwrite(q, 2, q_elems, f);
    fwrite(k, 2, pool_elems, f);
    fwrite(v, 2, pool_elems, f);
    fwrite(out, 2, q_elems, f);
    fwrite(lse, sizeof(float), (size_t)B * HQ, f);
    fclose(f);

    hipFree(dq); hipFree(dk); hipFree(dv); hipFree(dbt); hipFree(dlens); hipFree(dout); hipFree(dlse);
    hipFree(ws);
    hipStreamDestroy(stream);
    free(perm); free(bt); free(q); free(k); free(v); free(out); free(lse);
    return 0;
}
