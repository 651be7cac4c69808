/* Exhaustive check of the quotient method the store kernels use for absmax scales.
 *
 * For a row whose absmax is the bf16 value a, the scale is s = fl32(a / 127) and every value x of
 * the row is a bf16 value with |x| <= a.  The code is rint(fl32(x / s)) (IEEE division, ties to
 * even).  The kernels instead take r = fl32(1 / s) once per row and, per value, Markstein's
 * correction step (P. Markstein, "Computation of elementary functions on the IBM RISC System/6000
 * processor", IBM J. Res. Develop. 34(1), 1990): q0 = fl32(x r), e = fma(-q0, s, x) (x - q0 s, one
 * rounding), q = fma(e, r, q0); the code is rint(q).  q itself may differ from fl32(x / s) in its
 * last bit; this program checks that rint(q) never differs from rint(fl32(x / s)), for every
 * positive finite bf16 a with s >= 2^-100 (smaller scales take the IEEE division) and every finite
 * bf16 x with |x| <= a.  Prints the counts; exit status 1 on any mismatch.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#define NT 8

static float bf(uint32_t b) {
    uint32_t u = b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

typedef struct {
    int id;
    long long pairs, bad;
} job_t;

static void* run(void* p) {
    job_t* j = (job_t*)p;
    for (uint32_t ab = 1 + (uint32_t)j->id; ab < 0x7f80; ab += NT) {
        const float a = bf(ab);
        const float s = a / 127.0f;
        if (!(s >= 0x1p-100f)) continue;
        const float r = 1.0f / s;
        for (uint32_t xb = 0; xb < 0x10000; ++xb) {
            if (((xb >> 7) & 0xff) == 0xff) continue;
            const float x = bf(xb);
            if (fabsf(x) > a) continue;
            ++j->pairs;
            const float q0 = x * r;
            const float e = fmaf(-q0, s, x);
            const float q = fmaf(e, r, q0);
            if (rintf(q) != rintf(x / s)) ++j->bad;
        }
    }
    return NULL;
}

int main(void) {
    pthread_t t[NT];
    job_t j[NT];
    for (int i = 0; i < NT; ++i) {
        j[i].id = i;
        j[i].pairs = j[i].bad = 0;
        pthread_create(&t[i], NULL, run, &j[i]);
    }
    long long pairs = 0, bad = 0;
    for (int i = 0; i < NT; ++i) {
        pthread_join(t[i], NULL);
        pairs += j[i].pairs;
        bad += j[i].bad;
    }
    printf("pairs %lld mismatches %lld\n", pairs, bad);
    return bad != 0;
}
