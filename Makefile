# Build every native piece in-tree.
#   make            all libraries
#   make oracle     CPU oracle (test infrastructure)
#   make synth      input generators (host + device twin)
#   make lib        the product: libmoe_residency.so (HIP, gfx950)
#   make ceiling    HBM / host-link ceiling and copy-reference kernels
HIPCC    ?= /opt/rocm/bin/hipcc
CC       ?= gcc
ARCH     ?= gfx950
# Packed-FP32 VALU forms are disabled for all device code.
HIPFLAGS := --offload-arch=$(ARCH) -O3 -std=c++17 -fPIC -shared -Wall \
            -Xclang -target-feature -Xclang -packed-fp32-ops

PKG      := expert_weight_residency_amd
LIB_SRCS := $(wildcard $(PKG)/csrc/*.hip)
LIB_HDRS := $(wildcard $(PKG)/csrc/*.h) include/moe_residency.h

.PHONY: all oracle synth lib ceiling clean
all: oracle synth lib ceiling

oracle: oracle/liboracle.so
oracle/liboracle.so: oracle/moe_oracle.c
	$(CC) -O2 -ffp-contract=off -fno-fast-math -fopenmp -fPIC -shared -Wall -o $@ $<

synth: synth/libsynth.so synth/libsynth_dev.so
synth/libsynth.so: synth/synth.c
	$(CC) -O2 -fopenmp -fPIC -shared -Wall -o $@ $<
synth/libsynth_dev.so: synth/synth_dev.hip
	$(HIPCC) $(HIPFLAGS) -o $@ $<

lib: $(PKG)/libmoe_residency.so
$(PKG)/libmoe_residency.so: $(LIB_SRCS) $(LIB_HDRS)
	$(HIPCC) $(HIPFLAGS) -Iinclude -o $@ $(LIB_SRCS)

ceiling: ceiling/libceiling.so
ceiling/libceiling.so: ceiling/ceiling.hip
	$(HIPCC) $(HIPFLAGS) -o $@ $<

clean:
	rm -f oracle/liboracle.so synth/libsynth.so synth/libsynth_dev.so \
	      $(PKG)/libmoe_residency.so ceiling/libceiling.so
