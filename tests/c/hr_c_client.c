/*
 * hr_c_client.c -- a plain C99 user of libhr's C ABI (include/hr.h), with
 * the HIP runtime's C API and nothing else: no C++, no Python, no torch.
 *
 * Reads G contributions of N binary16 values from <in.bin> (G * N uint16,
 * rank-major), then
 *   1. folds them with hr_reduce_f16 into out0,
 *   2. if G == 2, runs one two-rank loopback hr_allreduce_f16 on two streams
 *      from hr_loopback_stream_create, into out1 (rank 0) and out2 (rank 1),
 *   3. if 2 <= G <= HR_MAX_WORLD, runs one hr_allreduce_group_f16 of all G
 *      ranks on a G-rank channel (one launch), into G more outputs,
 * and writes out0 [out1 out2] [G group outputs] to <out.bin>.  The test that builds and runs
 * it compares the outputs with the oracle.  Exit status: 0 on success.
 *
 * usage: hr_c_client G N in.bin out.bin
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "hr.h"

#define CHECK_HIP(x)                                                          \
    do {                                                                      \
        hipError_t e_ = (x);                                                  \
        if (e_ != hipSuccess) {                                               \
            fprintf(stderr, "%s:%d %s\n", __FILE__, __LINE__, #x);            \
            return 2;                                                         \
        }                                                                     \
    } while (0)
#define CHECK_HR(x)                                                           \
    do {                                                                      \
        hr_status s_ = (x);                                                   \
        if (s_ != HR_OK) {                                                    \
            fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x,         \
                    hr_status_str(s_));                                       \
            return 3;                                                         \
        }                                                                     \
    } while (0)

int main(int argc, char **argv)
{
    if (argc != 5) {
        fprintf(stderr, "usage: %s G N in.bin out.bin\n", argv[0]);
        return 1;
    }
    int G = atoi(argv[1]);
    size_t n = (size_t)strtoull(argv[2], NULL, 10);
    if (G < 1 || G > HR_MAX_G || n == 0)
        return 1;

    uint16_t *host = (uint16_t *)malloc((size_t)G * n * 2);
    uint16_t *res = (uint16_t *)malloc((size_t)(3 + G) * n * 2);
    FILE *f = fopen(argv[3], "rb");
    if (!host || !res || !f || fread(host, 2, (size_t)G * n, f) != (size_t)G * n)
        return 1;
    fclose(f);

    void *dev[HR_MAX_G];
    void *out[3 + HR_MAX_G];
    for (int g = 0; g < G; ++g) {
        CHECK_HIP(hipMalloc(&dev[g], n * 2));
        CHECK_HIP(hipMemcpy(dev[g], host + (size_t)g * n, n * 2, hipMemcpyHostToDevice));
    }
    for (int k = 0; k < 3 + G; ++k)
        CHECK_HIP(hipMalloc(&out[k], n * 2));

    hr_stream_t s0 = NULL, s1 = NULL;
    CHECK_HR(hr_loopback_stream_create(0, &s0));
    CHECK_HR(hr_reduce_f16((const void *const *)dev, G, out[0], n, s0));
    CHECK_HIP(hipStreamSynchronize((hipStream_t)s0));
    CHECK_HIP(hipMemcpy(res, out[0], n * 2, hipMemcpyDeviceToHost));
    size_t written = n;

    if (G == 2 && n <= HR_DEFAULT_MAX_NUMEL) {
        hr_channel ch = NULL;
        hr_channel_config cfg = {.device = 0, .world_size = 2, .timeout_us = 2000000u,
                                 .algorithm = HR_ALGO_AUTO};
        CHECK_HR(hr_create_channel(&cfg, &ch));
        CHECK_HR(hr_loopback_stream_create(0, &s1));
        CHECK_HR(hr_allreduce_f16(ch, 0, dev[0], out[1], n, s0));
        CHECK_HR(hr_allreduce_f16(ch, 1, dev[1], out[2], n, s1));
        CHECK_HIP(hipStreamSynchronize((hipStream_t)s0));
        CHECK_HIP(hipStreamSynchronize((hipStream_t)s1));
        CHECK_HR(hr_channel_status(ch));
        {   /* no wait timed out, so there is no timeout record */
            int trank = 0;
            uint32_t tmask = 1;
            uint64_t tcall = 1;
            CHECK_HR(hr_channel_timeout_info(ch, &trank, &tmask, &tcall));
            if (trank != -1 || tmask != 0 || tcall != 0) {
                fprintf(stderr, "unexpected timeout record: rank %d mask %u call %llu\n", trank,
                        (unsigned)tmask, (unsigned long long)tcall);
                return 4;
            }
        }
        CHECK_HIP(hipMemcpy(res + n, out[1], n * 2, hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(res + 2 * n, out[2], n * 2, hipMemcpyDeviceToHost));
        CHECK_HR(hr_destroy(ch));
        CHECK_HR(hr_loopback_stream_destroy(s1));
        written = 3 * n;
    }
    if (G >= 2 && G <= HR_MAX_WORLD) {
        hr_channel ch = NULL;
        hr_channel_config cfg = {.device = 0, .world_size = G, .max_numel = n, .timeout_us = 2000000u,
                                 .algorithm = HR_ALGO_AUTO};
        CHECK_HR(hr_create_channel(&cfg, &ch));
        CHECK_HR(hr_allreduce_group_f16(ch, (const void *const *)dev, (void *const *)(out + 3), n, s0));
        CHECK_HIP(hipStreamSynchronize((hipStream_t)s0));
        CHECK_HR(hr_channel_status(ch));
        for (int r = 0; r < G; ++r)
            CHECK_HIP(hipMemcpy(res + written + (size_t)r * n, out[3 + r], n * 2, hipMemcpyDeviceToHost));
        written += (size_t)G * n;
        CHECK_HR(hr_destroy(ch));
    }
    CHECK_HR(hr_loopback_stream_destroy(s0));

    f = fopen(argv[4], "wb");
    if (!f || fwrite(res, 2, written, f) != written)
        return 1;
    fclose(f);
    for (int g = 0; g < G; ++g)
        CHECK_HIP(hipFree(dev[g]));
    for (int k = 0; k < 3 + G; ++k)
        CHECK_HIP(hipFree(out[k]));
    free(host);
    free(res);
    return 0;
}
