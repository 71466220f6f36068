// abi_consumer.cpp -- a native program that uses the library through its C
// header alone: device memory from hipMalloc, no torch, no Python.  Test
// infrastructure: tests/test_gpu_native_consumer.py writes the inputs, runs this
// program, and compares what it writes back with the CPU oracle.
//
//   abi_consumer <in.bin> <out.bin>
//
// in.bin (little endian): int64 n_tensors; int64 numel[n_tensors]; int32 steps;
// float lr, beta1, beta2, eps, weight_decay, inv_loss_scale; then the whole
// list's param (bf16 bits), grad (bf16 bits), exp_avg, exp_avg_sq and master
// (fp32), each the tensors' elements one after another.
// out.bin: int32 step counter, int32 overflow flag of adamw_check_finite on the
// gradients, then param, exp_avg, exp_avg_sq and master after `steps` mixed
// steps of adamw_multi_tensor_step, in the input's layout.
//
// The tensors sit in one device buffer per stream with a 3-element gap after
// each, so tensors start at every 16-byte phase and the library peels heads.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "adamw.h"

#define CHECK_HIP(x)                                                                   \
    do {                                                                               \
        hipError_t e_ = (x);                                                           \
        if (e_ != hipSuccess) {                                                        \
            std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));        \
            std::exit(2);                                                              \
        }                                                                              \
    } while (0)

#define CHECK_ADAMW(x)                                                                 \
    do {                                                                               \
        adamw_status s_ = (x);                                                         \
        if (s_ != ADAMW_OK) {                                                          \
            std::fprintf(stderr, "%s failed (%d): %s\n", #x, (int)s_, adamw_last_error()); \
            std::exit(3);                                                              \
        }                                                                              \
    } while (0)

static void read_exact(FILE* f, void* p, size_t n)
{
    if (n && std::fread(p, 1, n, f) != n) {
        std::fprintf(stderr, "short read\n");
        std::exit(4);
    }
}

int main(int argc, char** argv)
{
    if (argc != 3) {
        std::fprintf(stderr, "usage: %s in.bin out.bin\n", argv[0]);
        return 1;
    }
    if (adamw_abi_version() != ADAMW_ABI_VERSION) {
        std::fprintf(stderr, "library ABI %d, header %d\n", adamw_abi_version(), ADAMW_ABI_VERSION);
        return 5;
    }
    FILE* in = std::fopen(argv[1], "rb");
    if (!in) return 4;
    int64_t nt = 0;
    read_exact(in, &nt, sizeof nt);
    std::vector<int64_t> numel((size_t)nt);
    read_exact(in, numel.data(), numel.size() * sizeof(int64_t));
    int32_t steps = 0;
    read_exact(in, &steps, sizeof steps);
    adamw_hparams hp;
    read_exact(in, &hp, sizeof hp);
    int64_t total = 0;
    for (int64_t n : numel) total += n;

    const int esz[5] = {2, 2, 4, 4, 4};   // param, grad, exp_avg, exp_avg_sq, master
    const int64_t kGap = 3;
    std::vector<int64_t> offset((size_t)nt);   // element offset of each tensor in the device buffers
    int64_t span = 0;
    for (int64_t i = 0; i < nt; ++i) {
        offset[(size_t)i] = span;
        span += numel[(size_t)i] + kGap;
    }
    std::vector<std::vector<unsigned char>> host(5);
    void* dev[5];
    for (int s = 0; s < 5; ++s) {
        host[(size_t)s].resize((size_t)(total * esz[s]));
        read_exact(in, host[(size_t)s].data(), host[(size_t)s].size());
        CHECK_HIP(hipMalloc(&dev[s], (size_t)((span + 8) * esz[s])));
        CHECK_HIP(hipMemset(dev[s], 0, (size_t)((span + 8) * esz[s])));
        int64_t src = 0;
        for (int64_t i = 0; i < nt; ++i) {
            const size_t bytes = (size_t)(numel[(size_t)i] * esz[s]);
            CHECK_HIP(hipMemcpy(static_cast<char*>(dev[s]) + offset[(size_t)i] * esz[s],
                                host[(size_t)s].data() + src, bytes, hipMemcpyHostToDevice));
            src += (int64_t)bytes;
        }
    }
    std::fclose(in);

    std::vector<std::vector<void*>> ptrs(5, std::vector<void*>((size_t)(nt ? nt : 1)));
    for (int s = 0; s < 5; ++s)
        for (int64_t i = 0; i < nt; ++i)
            ptrs[(size_t)s][(size_t)i] = static_cast<char*>(dev[s]) + offset[(size_t)i] * esz[s];
    adamw_tensor_list list;
    list.n_tensors = nt;
    list.numel = numel.data();
    for (int s = 0; s < 5; ++s) list.ptr[s] = ptrs[(size_t)s].data();
    list.shard_begin = 0;
    list.shard_end = -1;
    list.flat_mask = 0;

    int32_t* d_step = nullptr;
    int32_t* d_flag = nullptr;
    CHECK_HIP(hipMalloc(&d_step, sizeof(int32_t)));
    CHECK_HIP(hipMalloc(&d_flag, sizeof(int32_t)));
    CHECK_HIP(hipMemset(d_step, 0, sizeof(int32_t)));
    hipStream_t stream;
    CHECK_HIP(hipStreamCreate(&stream));
    for (int32_t t = 0; t < steps; ++t) CHECK_ADAMW(adamw_multi_tensor_step(ADAMW_MIXED, ADAMW_BF16, &list, &hp, d_step,
                                                                            nullptr, stream));
    CHECK_ADAMW(adamw_check_finite(ADAMW_BF16, &list, d_flag, stream));
    CHECK_HIP(hipStreamSynchronize(stream));

    int32_t step = 0, flag = 0;
    CHECK_HIP(hipMemcpy(&step, d_step, sizeof step, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(&flag, d_flag, sizeof flag, hipMemcpyDeviceToHost));
    FILE* out = std::fopen(argv[2], "wb");
    if (!out) return 4;
    std::fwrite(&step, sizeof step, 1, out);
    std::fwrite(&flag, sizeof flag, 1, out);
    const int written[4] = {0, 2, 3, 4};
    for (int s : written) {
        std::vector<unsigned char> back((size_t)(total * esz[s]));
        int64_t dst = 0;
        for (int64_t i = 0; i < nt; ++i) {
            const size_t bytes = (size_t)(numel[(size_t)i] * esz[s]);
            CHECK_HIP(hipMemcpy(back.data() + dst, static_cast<char*>(dev[s]) + offset[(size_t)i] * esz[s], bytes,
                                hipMemcpyDeviceToHost));
            dst += (int64_t)bytes;
        }
        std::fwrite(back.data(), 1, back.size(), out);
    }
    std::fclose(out);
    CHECK_HIP(hipStreamDestroy(stream));
    adamw_release_workspace();
    for (int s = 0; s < 5; ++s) CHECK_HIP(hipFree(dev[s]));
    CHECK_HIP(hipFree(d_step));
    CHECK_HIP(hipFree(d_flag));
    return 0;
}
