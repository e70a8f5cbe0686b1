/*
 * c_abi_demo.c -- drives libmoe through its C ABI alone (no Python, no
 * torch): the caller's side of include/moe.h written in plain C.
 *
 * Reads one layer's inputs from binary files in DIR (written by the GPU test
 * that runs this program), allocates every device buffer itself, packs the
 * expert weights into the fragment layout with moe_pack_weights, runs
 * moe_layer_forward with a workspace of moe_workspace_bytes bytes and
 * moe_layer_forward_noalloc, checks that the two outputs are bitwise equal,
 * and writes the first to DIR/out.bin.  Exit status 0 on success, 1 on any
 * failed call (the status string is printed).
 *
 *   DIR/shape.txt   hidden inter n_experts top_k n_slots n_shared T act seed
 *   DIR/h.bin       [T][hidden]              act (MOE_F16: 2 B, MOE_F32: 4 B)
 *   DIR/wr.bin      [n_experts (+1)][hidden] act (row n_experts: shared gate)
 *   DIR/gate.bin, up.bin [n_slots][inter][hidden]; down.bin [n_slots][hidden][inter]
 *   DIR/sh_gate.bin, sh_up.bin, sh_down.bin   the same per shared expert
 *   DIR/rep_off.bin int32 [n_experts + 1]; DIR/rep_slot.bin int32 [rep_off[E]]
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "moe.h"

static char g_dir[4096];

static void die(const char *what) {
    fprintf(stderr, "c_abi_demo: %s\n", what);
    exit(1);
}

static void check_hip(hipError_t e, const char *what) {
    if (e != hipSuccess) {
        fprintf(stderr, "c_abi_demo: %s: %s\n", what, hipGetErrorString(e));
        exit(1);
    }
}

static void check_moe(moe_status st, const char *what) {
    if (st != MOE_OK) {
        fprintf(stderr, "c_abi_demo: %s: %s\n", what, moe_status_str(st));
        exit(1);
    }
}

/* The whole file into host memory; *bytes gets its size. */
static void *read_file(const char *name, size_t *bytes) {
    char path[4200];
    snprintf(path, sizeof path, "%s/%s", g_dir, name);
    FILE *f = fopen(path, "rb");
    if (!f) die(path);
    fseek(f, 0, SEEK_END);
    long n = ftell(f);
    fseek(f, 0, SEEK_SET);
    void *p = malloc(n > 0 ? (size_t)n : 1);
    if (!p) die("out of host memory");
    if (n > 0 && fread(p, 1, (size_t)n, f) != (size_t)n) die(path);
    fclose(f);
    *bytes = (size_t)n;
    return p;
}

/* A file copied into a new device buffer of exactly `expect` bytes. */
static void *upload(const char *name, size_t expect) {
    size_t n = 0;
    void *h = read_file(name, &n);
    if (n != expect) {
        fprintf(stderr, "c_abi_demo: %s holds %zu bytes, expected %zu\n", name, n, expect);
        exit(1);
    }
    void *d = NULL;
    check_hip(hipMalloc(&d, expect > 0 ? expect : 16), "hipMalloc");
    if (expect) check_hip(hipMemcpy(d, h, expect, hipMemcpyHostToDevice), "hipMemcpy H2D");
    free(h);
    return d;
}

/* n_mats row-major [rows][cols] matrices uploaded, then packed into a second
 * device buffer (MOE_W_FRAG); the row-major copy is freed. */
static void *upload_packed(const char *name, int32_t dtype, int64_t n_mats, int32_t rows,
                           int32_t cols, size_t esize) {
    const size_t bytes = (size_t)n_mats * rows * cols * esize;
    void *src = upload(name, bytes);
    void *dst = NULL;
    check_hip(hipMalloc(&dst, bytes), "hipMalloc");
    check_moe(moe_pack_weights(dtype, n_mats, rows, cols, src, dst, NULL), "moe_pack_weights");
    check_hip(hipDeviceSynchronize(), "pack");
    check_hip(hipFree(src), "hipFree");
    return dst;
}

int main(int argc, char **argv) {
    if (argc != 2) die("usage: c_abi_demo DIR");
    snprintf(g_dir, sizeof g_dir, "%s", argv[1]);

    int H, I, E, K, S, NSH, T, act;
    unsigned long long seed;
    {
        char path[4200];
        snprintf(path, sizeof path, "%s/shape.txt", g_dir);
        FILE *f = fopen(path, "r");
        if (!f) die(path);
        if (fscanf(f, "%d %d %d %d %d %d %d %d %llu", &H, &I, &E, &K, &S, &NSH, &T, &act,
                   &seed) != 9)
            die("shape.txt: expected 9 numbers");
        fclose(f);
    }
    const size_t es = act == MOE_F32 ? 4 : 2;

    moe_shape shape;
    memset(&shape, 0, sizeof shape);
    shape.hidden = H;
    shape.inter = I;
    shape.n_experts = E;
    shape.top_k = K;
    shape.n_slots = S;
    shape.n_shared = NSH;
    shape.act = act;
    shape.dispatch = act;
    shape.flags = NSH > 0 ? MOE_F_SHARED : 0u;
    shape.w_layout = MOE_W_FRAG;

    moe_weights w;
    memset(&w, 0, sizeof w);
    w.w_router = upload("wr.bin", (size_t)(E + (NSH > 0)) * H * es);
    w.w_gate = upload_packed("gate.bin", act, S, I, H, es);
    w.w_up = upload_packed("up.bin", act, S, I, H, es);
    w.w_down = upload_packed("down.bin", act, S, H, I, es);
    if (NSH > 0) {
        w.sh_gate = upload_packed("sh_gate.bin", act, NSH, I, H, es);
        w.sh_up = upload_packed("sh_up.bin", act, NSH, I, H, es);
        w.sh_down = upload_packed("sh_down.bin", act, NSH, H, I, es);
    }

    size_t off_bytes = 0;
    int32_t *off_h = (int32_t *)read_file("rep_off.bin", &off_bytes);
    if (off_bytes != (size_t)(E + 1) * 4) die("rep_off.bin: expected E + 1 int32");
    const size_t nnz = (size_t)off_h[E];
    free(off_h);
    moe_slot_map map;
    map.rep_off = (const int32_t *)upload("rep_off.bin", (size_t)(E + 1) * 4);
    map.rep_slot = (const int32_t *)upload("rep_slot.bin", nnz * 4);
    map.seed = seed;

    void *h = upload("h.bin", (size_t)T * H * es);
    const size_t out_bytes = (size_t)T * H * es;
    void *out = NULL, *out2 = NULL, *ws = NULL;
    check_hip(hipMalloc(&out, out_bytes), "hipMalloc");
    check_hip(hipMalloc(&out2, out_bytes), "hipMalloc");
    const size_t ws_bytes = moe_workspace_bytes(&shape, T);
    if (ws_bytes == 0) die("moe_workspace_bytes refused the shape");
    check_hip(hipMalloc(&ws, ws_bytes), "hipMalloc");

    check_moe(moe_layer_forward(&shape, &w, &map, T, h, out, ws, ws_bytes, NULL),
              "moe_layer_forward");
    check_moe(moe_layer_forward_noalloc(&shape, &w, &map, T, h, out2, NULL),
              "moe_layer_forward_noalloc");
    check_hip(hipDeviceSynchronize(), "forward");

    void *o1 = malloc(out_bytes), *o2 = malloc(out_bytes);
    if (!o1 || !o2) die("out of host memory");
    check_hip(hipMemcpy(o1, out, out_bytes, hipMemcpyDeviceToHost), "hipMemcpy D2H");
    check_hip(hipMemcpy(o2, out2, out_bytes, hipMemcpyDeviceToHost), "hipMemcpy D2H");
    if (memcmp(o1, o2, out_bytes) != 0) die("moe_layer_forward_noalloc differs from moe_layer_forward");

    char path[4200];
    snprintf(path, sizeof path, "%s/out.bin", g_dir);
    FILE *f = fopen(path, "wb");
    if (!f || fwrite(o1, 1, out_bytes, f) != out_bytes) die(path);
    fclose(f);
    printf("c_abi_demo: %s T=%d H=%d I=%d E=%d K=%d S=%d shared=%d ok\n", moe_version(), T, H, I,
           E, K, S, NSH);
    return 0;
}
